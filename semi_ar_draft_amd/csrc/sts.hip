// Fitting the per-position confidence temperatures (sequential temperature
// scaling) by a grid search over candidate temperatures.
//
// [blog] "校准问题：原始置信度不可靠" and [summary] section 4: position by
// position, left to right, the temperature is the candidate whose scaled
// survival product prod_{i<k} sigmoid(l_i / T_i) * sigmoid(l_k / T) has the
// lowest expected calibration error (ECE) against the measured acceptance of
// positions 1..k, the earlier positions keeping the temperatures already
// chosen.  ECE uses M equal-width bins on [0, 1] (bin min(floor(S M), M-1)).
//
// The work is N samples x n_grid candidates of one scaled sigmoid, a bin
// decision and an accumulation per position: plain ALU work (an exponential
// and a reciprocal on the transcendental unit), with 4 bytes of logit read
// per sample and candidate row.  One launch per position does all of it,
// the last workgroup to finish choosing the temperature.  Two facts shape
// the kernel:
//  - a bin's share of the ECE is |sum over the bin of (label - score)| / N,
//    so one signed sum per (bin, candidate) is all that is kept; it is
//    accumulated as a 64-bit integer of 2^-30 units, so the sums, and the
//    choice of temperature, do not depend on the order of the atomics;
//  - the lanes of a wave are 64 candidates and the samples are broadcast to
//    them (LDS reads of one address), so lane g always adds into column g of
//    the histogram: the 64-bit LDS atomics of one instruction never share an
//    address.
#include <float.h>

#include "common.hpp"
#include "internal.hpp"

namespace dspark {
namespace {

constexpr float kStsScale = 1073741824.f;      // 2^30 fixed-point units per score unit
constexpr double kStsScaleD = 1073741824.0;

// sigmoid(x / T) with c = -log2(e) / T: 1 / (1 + 2^(x c))
__device__ __forceinline__ float scaled_sigmoid(float x, float c) {
  return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(x * c));
}

// ECE of every candidate from the global sums, which are read with
// agent-scope atomic loads and cleared for the next position; the first
// minimiser and its temperature.  Run by the last workgroup of a position's
// pass; `cell` is LDS of at least n_bins x n_grid doubles.
__device__ void select_position(const StsArgs& a, double* cell) {
  __shared__ double sv[256];
  __shared__ int si[256];
  const int ng = a.n_grid, nb = a.n_bins;
  const int cells = ng * nb;
  constexpr int kPer = kStsMaxCells / kStsThreads;
  unsigned long long v[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int i = threadIdx.x + kStsThreads * u;
    v[u] = i < cells ? __hip_atomic_load(&a.hist[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0ull;
  }
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int i = threadIdx.x + kStsThreads * u;
    if (i < cells) {
      const long long x = (long long)v[u];
      cell[i] = (double)(x < 0 ? -x : x);
      __hip_atomic_store(&a.hist[i], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  __syncthreads();
  double bv = DBL_MAX;
  int bi = 0x7fffffff;
  if (threadIdx.x < 256) {
    for (int g = threadIdx.x; g < ng; g += 256) {
      double s = 0.0;
      for (int m = 0; m < nb; ++m) s += cell[m * ng + g];
      const double e = a.N > 0 ? s / (kStsScaleD * (double)a.N) : 0.0;
      a.ece[(int64_t)(a.k - 1) * ng + g] = e;
      if (e < bv) {   // g grows along the loop: the first minimiser is kept
        bv = e;
        bi = g;
      }
    }
    sv[threadIdx.x] = bv;
    si[threadIdx.x] = bi;
  }
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) {
      const double ov = sv[threadIdx.x + w];
      const int oi = si[threadIdx.x + w];
      if (ov < sv[threadIdx.x] || (ov == sv[threadIdx.x] && oi < si[threadIdx.x])) {
        sv[threadIdx.x] = ov;
        si[threadIdx.x] = oi;
      }
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    int g = si[0];
    if (g < 0 || g >= ng) g = 0;   // unreachable: every ECE is finite
    a.T[a.k - 1] = a.grid[g];
    a.index[a.k - 1] = g;
    __hip_atomic_store(a.done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// One position: every wave takes blocks of 64 samples, stages each sample's
// (logit at k, prefix under the fitted earlier temperatures, label) in LDS,
// and then walks them one by one, all 64 lanes (NS slices of 64 candidates)
// scoring the same sample.  Sums of (label - score) per (bin, candidate)
// build up in LDS and are added into the global ones at the end; the last
// workgroup to finish selects the temperature.  Lanes past the last
// candidate add into a spare column that is never read.
template <int NS, int CELLS>
__global__ __launch_bounds__(kStsThreads) void sts_hist_impl(StsArgs a) {
  __shared__ unsigned long long h[CELLS + 64];
  __shared__ float4 samp[kStsWaves][64];
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int ng = a.n_grid, nb = a.n_bins;
  const int cells = nb * ng;
  for (int i = threadIdx.x; i < cells; i += kStsThreads) h[i] = 0ull;

  // the lane's candidates g = lane + 64 s: c = -log2(e) / T_g, and the LDS
  // byte address of (bin, g) = bin * mul + base
  float cg[NS];
  unsigned mul[NS], base[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int g = lane + 64 * s;
    if (g < ng) {
      const float t = a.grid[g];
      if (!(t > 0.f) || !(t <= FLT_MAX)) atomicOr(a.err, kErrGrid);
      cg[s] = -kLog2e / t;
      mul[s] = (unsigned)ng * 8u;
      base[s] = (unsigned)g * 8u;
    } else {
      cg[s] = 0.f;
      mul[s] = 0u;
      base[s] = (unsigned)(CELLS + lane) * 8u;
    }
  }
  __syncthreads();

  // bin = floor(S * M * (1 - 2^-22)): below M for every S <= 1, so no clamp
  // is needed; it differs from floor(S * M) only for scores within 2.4e-7
  // below a bin edge, inside the fp32 error of S itself
  const float fM = (float)nb * (1.f - 0x1p-22f);
  const int k = a.k;
  const int64_t N = a.N;
  char* hb = reinterpret_cast<char*>(h);
  for (int64_t b0 = ((int64_t)blockIdx.x * kStsWaves + wid) * 64; b0 < N;
       b0 += (int64_t)gridDim.x * kStsWaves * 64) {
    const int64_t n = b0 + lane;
    float p = 0.f, l = 0.f, ys = 0.f;   // prefix, logit at k, label x 2^30
    if (n < N) {
      const float* row = a.logit + n * a.stride;
      float pre = 1.f;
      for (int i = 0; i < k - 1; ++i) pre *= scaled_sigmoid(row[i], -kLog2e / a.T[i]);
      p = pre;
      l = row[k - 1];
      int len = a.len[n];
      if (len < 0 || len > a.gamma) {
        atomicOr(a.err, kErrLen);
        len = len < 0 ? 0 : a.gamma;
      }
      ys = len >= k ? kStsScale : 0.f;
    }
    // the wave's own staging row: its LDS accesses complete in order.  Per
    // draft: logit, prefix x 2^30, label x 2^30, prefix x M'
    samp[wid][lane] = make_float4(l, p * kStsScale, ys, p * fM);
    __builtin_amdgcn_wave_barrier();
    // Groups of four drafts, double-buffered: the next group's broadcast
    // reads are issued before this group's atomics, so they do not wait
    // behind them in the wave's in-order LDS queue.  A group is scored phase
    // by phase (independent exponentials, then reciprocals, ...), so the
    // transcendental latencies overlap.  A sample past N has prefix 0, scores
    // 0 with label 0 and so adds 0 (into bin 0).  With sg = sigmoid(l / T)
    // and S = prefix * sg: q = (label - S) x 2^30 and bin = floor(S M').
    float4 v[4], vn[4] = {};
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = samp[wid][u];
    for (int j0 = 0; j0 < 64; j0 += 4) {
      if (j0 + 4 < 64) {
#pragma unroll
        for (int u = 0; u < 4; ++u) vn[u] = samp[wid][j0 + 4 + u];
      }
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        float sg[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) sg[u] = __builtin_amdgcn_exp2f(v[u].x * cg[s]);
#pragma unroll
        for (int u = 0; u < 4; ++u) sg[u] = __builtin_amdgcn_rcpf(1.f + sg[u]);
        unsigned addr[4];
        int q[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const unsigned bin = (unsigned)(sg[u] * v[u].w);
          q[u] = (int)fmaf(sg[u], -v[u].y, v[u].z);            // (label - S) in 2^-30 units
          addr[u] = __umul24(bin, mul[s]) + base[s];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
          atomicAdd(reinterpret_cast<unsigned long long*>(hb + addr[u]), (unsigned long long)(long long)q[u]);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = vn[u];
    }
    __builtin_amdgcn_wave_barrier();
  }
  __syncthreads();
  for (int i = threadIdx.x; i < cells; i += kStsThreads) {
    const unsigned long long v = h[i];
    if (v) atomicAdd(&a.hist[i], v);
  }
  // the last workgroup to finish turns the sums into the position's ECE
  // table and temperature.  The sums are device-scope atomics, performed
  // where every XCD sees them: each wave waits until its own have been
  // acknowledged before the workgroup is counted, and the last workgroup
  // reads them back with agent-scope atomic loads.  (Cache write-back and
  // invalidation fences are not needed for that, and cost 4x the pass.)
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  __shared__ int is_last;
  if (threadIdx.x == 0)
    is_last = __hip_atomic_fetch_add(a.done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == gridDim.x - 1;
  __syncthreads();
  if (!is_last) return;
  select_position(a, reinterpret_cast<double*>(h));
}

}  // namespace

const void* sts_hist_kernel(int n_slices, int cells) {
  // histogram of at most 1024 cells: 12.7 KB of LDS per workgroup instead of 37 KB
  if (cells <= 1024) {
    switch (n_slices) {
      case 1: return (const void*)sts_hist_impl<1, 1024>;
      case 2: return (const void*)sts_hist_impl<2, 1024>;
      case 3: return (const void*)sts_hist_impl<3, 1024>;
      default: return (const void*)sts_hist_impl<4, 1024>;
    }
  }
  switch (n_slices) {
    case 1: return (const void*)sts_hist_impl<1, kStsMaxCells>;
    case 2: return (const void*)sts_hist_impl<2, kStsMaxCells>;
    case 3: return (const void*)sts_hist_impl<3, kStsMaxCells>;
    default: return (const void*)sts_hist_impl<4, kStsMaxCells>;
  }
}

}  // namespace dspark
