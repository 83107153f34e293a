// Hardware-aware prefix scheduler: greedy admission with early stop, in one
// workgroup.
//
// [blog] "硬件感知前缀调度器" steps 1-4: build every (request, length)
// candidate with its survival a, sort from high to low, admit greedily while
// tracking Theta = tau * SPS, stop once Theta stops increasing; [summary]
// section 4 (expected accepted tokens times the steps/s of the resulting
// batch, read from a profiled table).
//
// Greedy admission in sorted order makes the admitted set after n steps the
// top-n candidates, so every Theta_n is known once the sorted prefix sums
// S_n are: Theta_n = (B + S_n) * SPS[B + n - 1].  The sequential loop of the
// definition becomes sort -> scan -> first n with Theta_n <= Theta_{n-1}.
// Keys are 64-bit: (~bits(a)) << 32 | (b * gamma + j - 1), so an ascending
// sort orders a descending, then request, then position.  Sums and Theta are
// float64: sums of float32 survivals are exact in float64 for any realistic
// spread of magnitudes, so the order of the scan does not change them.
#include "common.hpp"
#include "internal.hpp"

namespace dspark {
namespace {

constexpr int kSchedKeys = 4096;   // B * gamma <= kSchedKeys
constexpr int kPerThread = kSchedKeys / kSchedThreads;

__device__ __forceinline__ float key_value(uint64_t k) {
  return __uint_as_float(~(uint32_t)(k >> 32));
}

// Keys of the survivals in src, padded with the largest key, sorted
// ascending in LDS (bitonic).
__device__ void sort_keys(uint64_t* keys, const float* src, int n, int n_pad) {
  const int tid = threadIdx.x;
  for (int i = tid; i < n_pad; i += kSchedThreads) {
    uint64_t key = ~0ull;
    if (i < n) {
      float v = src[i];
      v = (v > 0.0f) ? v : 0.0f;    // NaN, negatives and -0 read as +0
      key = ((uint64_t)(~__float_as_uint(v)) << 32) | (uint32_t)i;
    }
    keys[i] = key;
  }
  __syncthreads();
  for (int size = 2; size <= n_pad; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int t = tid; t < (n_pad >> 1); t += kSchedThreads) {
        const int i = 2 * t - (t & (stride - 1));
        const int jx = i + stride;
        const uint64_t ki = keys[i], kj = keys[jx];
        const bool up = (i & size) == 0;
        if ((ki > kj) == up) {
          keys[i] = kj;
          keys[jx] = ki;
        }
      }
      __syncthreads();
    }
  }
}

// Exclusive prefix (float64) of this thread's segment of the sorted list.
__device__ double segment_prefix(const uint64_t* keys, double* wave_tot, int n, int p0, int seg) {
  const int tid = threadIdx.x;
  double part = 0.0;
  for (int e = 0; e < seg; ++e) {
    const int p = p0 + e;
    if (p < n) part += (double)key_value(keys[p]);
  }
  const int lane = tid & 63, wid = tid >> 6;
  double inc = part;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const double o = __shfl_up(inc, d, 64);
    if (lane >= d) inc += o;
  }
  if (lane == 63) wave_tot[wid] = inc;
  __syncthreads();
  double wave_pre = 0.0;
  for (int w = 0; w < wid; ++w) wave_pre += wave_tot[w];
  double excl = __shfl_up(inc, 1, 64);
  if (lane == 0) excl = 0.0;
  return wave_pre + excl;
}

// (Theta, n) pairs: larger Theta first, then smaller n.
__device__ __forceinline__ bool theta_beats(double t2, int n2, double t1, int n1) {
  return t2 > t1 || (t2 == t1 && n2 < n1);
}

// ASYNC = 0: the synchronous rule (admit in sorted order, stop at the first
// n with Theta_n <= Theta_{n-1}).  ASYNC = 1: the count n* is the first
// maximum of Theta_n over the sorted historical survivals (no early stop),
// and the admitted candidates are the top n* of the current survivals.
template <int ASYNC>
__global__ __launch_bounds__(kSchedThreads) void schedule_impl(const SchedArgs a) {
  __shared__ uint64_t keys[kSchedKeys];
  __shared__ double wave_tot[kSchedThreads / 64];
  __shared__ double wave_th[kSchedThreads / 64];
  __shared__ int wave_n[kSchedThreads / 64];
  __shared__ int first_stop;
  __shared__ int s_nsel;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wid = tid >> 6;
  const int n = a.B * a.gamma;
  int n_pad = 2;
  while (n_pad < n) n_pad <<= 1;
  if (tid == 0) first_stop = 0x7fffffff;
  sort_keys(keys, ASYNC ? a.surv_hist : a.surv, n, n_pad);
  // each thread: a contiguous segment of the sorted list
  const int seg = (n_pad >= kSchedThreads) ? n_pad / kSchedThreads : 1;
  const int p0 = tid * seg;
  double S = segment_prefix(keys, wave_tot, n, p0, seg);
  const double Bd = (double)a.B;
  const double theta0 = Bd * (double)a.sps[a.B - 1];
  const int n_max = min(n, a.n_sps - a.B);
  int bidx[kPerThread];
  double S_at[kPerThread];
  double best_th = -1.0;
  int best_n = 0x7fffffff;
  for (int e = 0; e < seg; ++e) {
    const int p = p0 + e;
    bidx[e] = -1;
    S_at[e] = 0.0;
    if (p >= n) continue;
    const uint64_t key = keys[p];
    const double S_prev = S;
    S = S + (double)key_value(key);
    S_at[e] = S;
    bidx[e] = (int)((uint32_t)key) / a.gamma;
    if (p < n_max) {
      const int N = a.B + p + 1;
      const double th = (Bd + S) * (double)a.sps[N - 1];
      if (ASYNC) {
        if (theta_beats(th, p + 1, best_th, best_n)) {
          best_th = th;
          best_n = p + 1;
        }
      } else {
        const double th_prev = (p == 0) ? theta0 : (Bd + S_prev) * (double)a.sps[N - 2];
        if (th <= th_prev) atomicMin(&first_stop, p);
      }
    }
  }
  if (ASYNC) {
    // argmax over n (n = 0 is Theta_0): within waves, then across them
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const double t2 = __shfl_xor(best_th, d, 64);
      const int n2 = __shfl_xor(best_n, d, 64);
      if (theta_beats(t2, n2, best_th, best_n)) {
        best_th = t2;
        best_n = n2;
      }
    }
    if (lane == 0) {
      wave_th[wid] = best_th;
      wave_n[wid] = best_n;
    }
    __syncthreads();
    if (tid == 0) {
      double bt = theta0;
      int bn = 0;
      for (int w = 0; w < kSchedThreads / 64; ++w)
        if (theta_beats(wave_th[w], wave_n[w], bt, bn)) {
          bt = wave_th[w];
          bn = wave_n[w];
        }
      s_nsel = bn;
      *a.theta = bt;
      *a.n_selected = bn;
    }
    __syncthreads();
    // rank the current survivals; the admitted set is their top n*
    sort_keys(keys, a.surv, n, n_pad);
    for (int e = 0; e < seg; ++e) {
      const int p = p0 + e;
      bidx[e] = p < n ? (int)((uint32_t)keys[p]) / a.gamma : -1;
    }
  } else {
    __syncthreads();
    const int nsel = min(first_stop, n_max);
    // Theta at the admitted set
    if (nsel == 0) {
      if (tid == 0) *a.theta = theta0;
    } else {
      for (int e = 0; e < seg; ++e) {
        if (p0 + e == nsel - 1) *a.theta = (Bd + S_at[e]) * (double)a.sps[a.B + nsel - 1];
      }
    }
    if (tid == 0) {
      *a.n_selected = nsel;
      s_nsel = nsel;
    }
  }
  // K_b: count admitted candidates per request (reusing the key storage)
  __syncthreads();
  const int nsel = s_nsel;
  int* counts = reinterpret_cast<int*>(keys);
  __syncthreads();
  for (int i = tid; i < a.B; i += kSchedThreads) counts[i] = 0;
  __syncthreads();
  for (int e = 0; e < seg; ++e) {
    if (p0 + e < nsel) atomicAdd(&counts[bidx[e]], 1);
  }
  __syncthreads();
  for (int i = tid; i < a.B; i += kSchedThreads) a.K[i] = counts[i];
}

}  // namespace

const void* schedule_kernel(int async) {
  return async ? (const void*)&schedule_impl<1> : (const void*)&schedule_impl<0>;
}

}  // namespace dspark
