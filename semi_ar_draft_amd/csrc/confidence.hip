// Confidence head with per-position temperature scaling, and survival
// products.
//
// [blog] "置信度头：预测自己的命运": c_k = sigmoid of a linear map of
// [h_k ; emb(x_{k-1})]; [blog] "校准问题：原始置信度不可靠": per-position
// temperature T_k applied to the logit; [teardown] "硬件感知前缀调度器" and
// [summary] section 4: survival a_j = prod_{i<=j} c_i.
//
// The head is a GEMV over 2 x 4096 bf16 values per (request, position): it is
// bound by HBM (h and the gathered embedding rows).  One launch does both
// the confidences and the survival products: a request's positions share a
// workgroup, so the prefix product needs no second kernel.
#include "common.hpp"
#include "internal.hpp"

namespace dspark {
namespace {

constexpr int kConfThreads = 1024;

// One workgroup per request.  Two waves per position: wave 2 (k - 1) takes
// the h_k half of the dot product, wave 2 (k - 1) + 1 the E[x_{k-1}] half;
// a lane takes every 64th 16-byte chunk, all eight of a round in flight at
// once, and the lanes reduce in a fixed shuffle tree.  The confidences and
// their prefix products are then formed in position order.
constexpr int kConfUnroll = 8;

__device__ __forceinline__ float half_dot(const uint16_t* x, const uint16_t* w, int n8, int lane) {
  float acc = 0.f;
  for (int i0 = lane; i0 < n8; i0 += 64 * kConfUnroll) {
    uint4 xv[kConfUnroll], wv[kConfUnroll];
#pragma unroll
    for (int u = 0; u < kConfUnroll; ++u) {
      const int i = i0 + 64 * u;
      xv[u] = i < n8 ? *reinterpret_cast<const uint4*>(x + 8 * i) : make_uint4(0u, 0u, 0u, 0u);
      wv[u] = i < n8 ? *reinterpret_cast<const uint4*>(w + 8 * i) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < kConfUnroll; ++u) {
      const uint32_t xs[4] = {xv[u].x, xv[u].y, xv[u].z, xv[u].w};
      const uint32_t ws[4] = {wv[u].x, wv[u].y, wv[u].z, wv[u].w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        acc = __builtin_fmaf(__uint_as_float(xs[t] << 16), __uint_as_float(ws[t] << 16), acc);
        acc = __builtin_fmaf(__uint_as_float(xs[t] & 0xFFFF0000u), __uint_as_float(ws[t] & 0xFFFF0000u), acc);
      }
    }
  }
  return acc;
}

// Confidences and survival products of request b; previous tokens from
// `toks` (shared memory, [gamma]) when given, else from a.tokens.
__device__ __forceinline__ void confidence_request(const ConfArgs& a, int b, const int* toks) {
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  __shared__ float part[kMaxGamma][2];
  __shared__ float val[kMaxGamma];
  for (int w = wid; w < 2 * a.gamma; w += kConfThreads / 64) {
    const int k = (w >> 1) + 1;
    float acc;
    if ((w & 1) == 0) {
      acc = half_dot(a.h + ((int64_t)b * a.gamma + k - 1) * a.dh, a.wc, a.dh >> 3, lane);
    } else {
      int prev = (k == 1) ? a.anchor[b] : toks ? toks[k - 2] : a.tokens[(int64_t)b * a.gamma + k - 2];
      if ((unsigned)prev >= (unsigned)a.V) {
        if (lane == 0) atomicOr(a.err, kErrToken);
        prev = 0;
      }
      acc = half_dot(a.E + (int64_t)prev * a.de, a.wc + a.dh, a.de >> 3, lane);
    }
#pragma unroll
    for (int mask = 1; mask < 64; mask <<= 1) acc += shfl_xor(acc, mask);
    if (lane == 0) part[k - 1][w & 1] = acc;
  }
  __syncthreads();
  if ((int)threadIdx.x < a.gamma) {
    const int k = threadIdx.x + 1;
    const float l = (part[k - 1][0] + part[k - 1][1]) + a.bc;
    const float T = a.sts ? a.sts[k - 1] : 1.0f;
    const float c = 1.0f / (1.0f + __expf(-l / T));
    a.conf[(int64_t)b * a.gamma + k - 1] = c;
    val[k - 1] = c;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float sv = 1.0f;
    for (int k = 0; k < a.gamma; ++k) {
      sv *= val[k];
      a.surv[(int64_t)b * a.gamma + k] = sv;
    }
  }
}

__global__ __launch_bounds__(kConfThreads) void confidence_impl(const ConfArgs a) {
  confidence_request(a, blockIdx.x, nullptr);
}

// The draft's merge and the confidence head in one launch, one 384-thread
// workgroup per (request b, position k).  Waves 0-3 merge position k's chunk
// partials exactly as the draft combine does (thread t folds chunks t,
// t + 256, ... in turn, each wave reduces by a butterfly, the four wave
// results are merged in order) and write x_k, the log-normaliser and y at
// x_k, and the position's slot groups are cleared.  Meanwhile waves 4 and 5
// form the confidence of the position whose previous token is x_k (position
// k + 1; the workgroup of the last position takes position 1, whose previous
// token is the anchor): wave 4 the h half of its dot product, wave 5 the
// embedding half.  Wave 5 takes x_k from the maximum of the position's slot
// groups, which orders (key, index) pairs as the merge does, so its row is
// read alongside the merge (without slot groups it waits for the merge).
// The request's last workgroup to finish (a counter per request; confidences
// stored and read with agent-scope atomics) forms the survival products in
// position order and clears the counter.
constexpr int kConfMergeThreads = 384;

__device__ __forceinline__ float conf_e_half(const ConfArgs& f, int prev, int lane) {
  if ((unsigned)prev >= (unsigned)f.V) {
    if (lane == 0) atomicOr(f.err, kErrToken);
    prev = 0;
  }
  float acc = half_dot(f.E + (int64_t)prev * f.de, f.wc + f.dh, f.de >> 3, lane);
#pragma unroll
  for (int mask = 1; mask < 64; mask <<= 1) acc += shfl_xor(acc, mask);
  return acc;
}

__global__ __launch_bounds__(kConfMergeThreads) void conf_merge_impl(const ConfMergeArgs a) {
  const CombineArgs& m = a.m;
  const ConfArgs& f = a.f;
  const int b = blockIdx.x;
  const int k = blockIdx.y + 1;
  const int kc = k < f.gamma ? k + 1 : 1;   // the confidence formed here
  const bool early = kc == 1 || m.best;     // its previous token known before the merge
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  __shared__ DraftPart red[4];
  __shared__ float part;
  __shared__ int s_tok;
  float acc = 0.f;
  if (wid < 4) {
    DraftPart p{-INFINITY, 0.f, -INFINITY, 0.f, 0x7fffffff};
    const int64_t base = ((int64_t)(k - 1) * m.B + b) * m.n_vc;
    for (int i = threadIdx.x; i < m.n_vc; i += 256) {
      const float4 q = m.pf[base + i];
      part_merge(p, DraftPart{q.x, q.y, q.z, q.w, m.pi[base + i].x});
    }
#pragma unroll
    for (int mask = 1; mask < 64; mask <<= 1) part_merge(p, part_shfl(p, mask));
    if (lane == 0) red[wid] = p;
  } else if (wid == 4) {
    acc = half_dot(f.h + ((int64_t)b * f.gamma + kc - 1) * f.dh, f.wc, f.dh >> 3, lane);
#pragma unroll
    for (int mask = 1; mask < 64; mask <<= 1) acc += shfl_xor(acc, mask);
    if (lane == 0) part = acc;
  } else if (early) {
    int prev;
    if (kc == 1) {
      prev = f.anchor[b];
    } else {
      unsigned long long v = 0ull;
      if (lane < kBestGroups) v = m.best[((int64_t)(k - 1) * kBestGroups + lane) * m.B + b];
      // over the whole wave: every lane reads its share of the row at x_k
#pragma unroll
      for (int mask = 1; mask < 64; mask <<= 1) {
        const unsigned long long o = __shfl_xor(v, mask, 64);
        v = o > v ? o : v;
      }
      prev = best_index(v);
    }
    acc = conf_e_half(f, prev, lane);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    DraftPart p = red[0];
#pragma unroll
    for (int w = 1; w < 4; ++w) part_merge(p, red[w]);
    int idx = p.idx;
    if ((unsigned)idx >= (unsigned)m.V) {
      atomicOr(m.err, kErrToken);
      idx = 0;
    }
    const int64_t o = (int64_t)b * m.gamma + k - 1;
    m.tokens[o] = idx;
    m.lse[o] = (p.m + fast_log2(p.s)) * kLn2;
    m.ytok[o] = m.greedy ? p.key : p.zb;   // sampling partials carry y itself
    s_tok = idx;
  }
  if (m.bar && b == 0 && k == 1 && threadIdx.x == 0) *m.bar = 0u;   // grid barrier of the whole-draft kernel
  if (m.chain && b == 0 && k == 1 && threadIdx.x < 97)   // chained draft counters
    m.chain[threadIdx.x == 0 ? 0 : 31 + threadIdx.x] = 0u;
  if (m.best && threadIdx.x < kBestGroups) {   // read above, before this barrier
    unsigned long long* slot = m.best + ((int64_t)(k - 1) * kBestGroups + threadIdx.x) * m.B + b;
    __hip_atomic_store(slot, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (!early) {   // uniform over the workgroup
    __syncthreads();
    if (wid == 5) acc = conf_e_half(f, s_tok, lane);
  }
  if (wid == 5 && lane == 0) {
    const float l = (part + acc) + f.bc;
    const float T = f.sts ? f.sts[kc - 1] : 1.0f;
    const float c = 1.0f / (1.0f + __expf(-l / T));
    float* conf = f.conf + (int64_t)b * f.gamma;
    __hip_atomic_store(reinterpret_cast<unsigned*>(conf + kc - 1), __float_as_uint(c), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(0xF70);                   // stored before the request counts it
    const unsigned before = __hip_atomic_fetch_add(a.cnt + b, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (before == (unsigned)f.gamma - 1u) {
      // every confidence of the request is in: survival products in position order
      __hip_atomic_store(a.cnt + b, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      float sv = 1.0f;
      for (int j = 0; j < f.gamma; ++j) {
        sv *= __uint_as_float(__hip_atomic_load(reinterpret_cast<const unsigned*>(conf + j), __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT));
        f.surv[(int64_t)b * f.gamma + j] = sv;
      }
    }
  }
}

}  // namespace

const void* confidence_kernel() { return (const void*)&confidence_impl; }
const void* conf_merge_kernel() { return (const void*)&conf_merge_impl; }

}  // namespace dspark
