// Verification: streaming passes over the target rows of every request, then
// one wave per request that walks its positions in order.  Rows are taken in
// windows (rows 1-2, then the rest): a row after a request's first rejection
// is never needed, so the later window only reads rows of requests that have
// accepted every position so far.
//
// [blog] "形式化定义": the target scores every drafted position in one pass,
// positions are checked in order, the first rejected one is replaced by a
// target token and the rest dropped, so the output law is the target's.
// Row statistics (log-sum-exp of t/T; greedy arg-max; the bonus row's
// group-race draw from exp(t/T)) need the whole vocabulary and are formed here; the accept tests need
// only t at the drafted token, read directly by the decision kernel.  The
// residual draw at the first rejection reuses the MFMA sweep (sweep.hip).
#include "common.hpp"
#include "internal.hpp"

namespace dspark {
namespace {

constexpr int kRowsThreads = 256;

__device__ __forceinline__ int clamp_k(const int32_t* K, int b, int gamma, int32_t* err, bool report) {
  if (!K) return gamma;
  int kb = K[b];
  if (kb < 0 || kb > gamma) {
    if (report) atomicOr(err, kErrK);
    kb = kb < 0 ? 0 : gamma;
  }
  return kb;
}

struct RowState {
  float m, s, key;
  int idx;
};

__device__ __forceinline__ void row_merge(RowState& a, const RowState& b) {
  softmax_merge(a.m, a.s, b.m, b.s);
  if (key_beats(b.key, b.idx, a.key, a.idx)) {
    a.key = b.key;
    a.idx = b.idx;
  }
}

// KEYMODE 0: no key, 1: arg-max of t, 2: group-race draw from exp(t/T) (the
// four values of a float4 form one aligned race group).
template <int KEYMODE>
__device__ __forceinline__ void row_fold(RowState& st, const float4 x, int v0, float s2, uint32_t klo,
                                         uint32_t khi) {
  const float xv[4] = {x.x, x.y, x.z, x.w};
  float y2[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) y2[i] = xv[i] * s2;
  const float mt = fmaxf(fmaxf(y2[0], y2[1]), fmaxf(y2[2], y2[3]));
  const float mn = fmaxf(st.m, mt);
  float e[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) e[i] = fast_exp2(y2[i] - mn);
  const float S = (e[0] + e[1]) + (e[2] + e[3]);
  st.s = st.s * fast_exp2(st.m - mn) + S;
  st.m = mn;
  if constexpr (KEYMODE == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (xv[i] > st.key) {
        st.key = xv[i];
        st.idx = v0 + i;
      }
    }
  } else if constexpr (KEYMODE == 2) {
    const float E = -fast_log2(hash_uniform(elem_hash(klo, khi, (uint32_t)v0)));
    if (E < S * fast_exp2(mn - st.key)) {
      const float key = fast_log2(S) + mn - fast_log2(E);
      if (key > st.key) {
        const float c = hash_uniform(elem_hash(klo, khi, (uint32_t)(v0 + 1))) * S;
        st.key = key;
        st.idx = v0 + group_pick(c, e[0], e[1], e[2], e[3]);
      }
    }
  }
}

template <int KEYMODE>
__device__ __forceinline__ void row_sweep(RowState& st, const float4* p, int c0, int c1, float s2,
                                          uint32_t klo, uint32_t khi) {
  int i = c0 + (int)threadIdx.x;
  // four independent 16-byte loads in flight per thread
  for (; i + 3 * kRowsThreads < c1; i += 4 * kRowsThreads) {
    const float4 x0 = p[i];
    const float4 x1 = p[i + kRowsThreads];
    const float4 x2 = p[i + 2 * kRowsThreads];
    const float4 x3 = p[i + 3 * kRowsThreads];
    row_fold<KEYMODE>(st, x0, 4 * i, s2, klo, khi);
    row_fold<KEYMODE>(st, x1, 4 * (i + kRowsThreads), s2, klo, khi);
    row_fold<KEYMODE>(st, x2, 4 * (i + 2 * kRowsThreads), s2, klo, khi);
    row_fold<KEYMODE>(st, x3, 4 * (i + 3 * kRowsThreads), s2, klo, khi);
  }
  for (; i < c1; i += kRowsThreads) row_fold<KEYMODE>(st, p[i], 4 * i, s2, klo, khi);
}

__global__ __launch_bounds__(kRowsThreads) void verify_rows_impl(const RowsArgs a) {
  const int nrows = a.hi - a.lo + 1;
  const int chunk = blockIdx.x;
  const int b = blockIdx.y / nrows;
  const int k = a.lo + blockIdx.y % nrows;
  if (a.vstate && a.vstate[b].y == 0) return;   // request already decided
  const int kb = clamp_k(a.K, b, a.gamma, a.err, chunk == 0 && k == 1 && threadIdx.x == 0);
  if (k > kb + 1) return;
  const int row = b * (a.gamma + 1) + (k - 1);
  const bool bonus = (k == kb + 1);
  const float4* p = reinterpret_cast<const float4*>(a.T + (int64_t)b * a.tsb + (int64_t)(k - 1) * a.tsk);
  const int nv4 = a.V >> 2;
  const int c0 = (int)((int64_t)nv4 * chunk / a.n_chunks);
  const int c1 = (int)((int64_t)nv4 * (chunk + 1) / a.n_chunks);
  RowState st{-INFINITY, 0.f, -INFINITY, 0x7fffffff};
  if (a.greedy) {
    row_sweep<1>(st, p, c0, c1, a.s2, 0, 0);
  } else if (bonus) {
    const uint32_t req = a.req ? a.req[b] : (uint32_t)b;
    const uint64_t key = stream_key(a.seed, req, (uint32_t)k, kBonus);
    row_sweep<2>(st, p, c0, c1, a.s2, (uint32_t)key, (uint32_t)(key >> 32));
  } else {
    row_sweep<0>(st, p, c0, c1, a.s2, 0, 0);
  }
  // wave reduction, then across the four waves in a fixed order
#pragma unroll
  for (int mask = 1; mask < 64; mask <<= 1) {
    RowState o{shfl_xor(st.m, mask), shfl_xor(st.s, mask), shfl_xor(st.key, mask),
               shfl_xor(st.idx, mask)};
    row_merge(st, o);
  }
  __shared__ RowState red[kRowsThreads / 64];
  const int wid = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wid] = st;
  __syncthreads();
  if (threadIdx.x == 0) {
    RowState acc = red[0];
#pragma unroll
    for (int w = 1; w < kRowsThreads / 64; ++w) row_merge(acc, red[w]);
    const int64_t o = (int64_t)row * a.pstride + chunk;
    a.pf[o] = make_float4(acc.m, acc.s, acc.key, 0.f);
    a.pi[o] = acc.idx;
  }
}

constexpr int kMaxGamma = 32;

// One wave per request: finish the statistics of the rows of this window,
// then continue the request's accept decisions in order.  Writes the kept
// drafts, the compensation / bonus token when it is known here, the residual
// request otherwise; a request that kept every row of the window and has
// rows left stays pending for the next window.
__global__ __launch_bounds__(64) void verify_decide_impl(const DecideArgs a) {
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  int A = 0;
  int start = 1;
  if (!a.first) {
    const int2 vs = a.vstate[b];
    if (vs.y == 0) return;
    A = vs.x;
    start = vs.y;
  }
  const int kb = clamp_k(a.K, b, a.gamma, a.err, false);
  const int last = min(a.hi, kb + 1);
  __shared__ float s_lt[kMaxGamma + 1];
  __shared__ int s_star[kMaxGamma + 1];
  for (int k = start; k <= last; ++k) {
    const int64_t base = ((int64_t)b * (a.gamma + 1) + (k - 1)) * a.pstride;
    RowState st{-INFINITY, 0.f, -INFINITY, 0x7fffffff};
    for (int c = lane; c < a.n_chunks; c += 64) {
      const float4 p = a.pf[base + c];
      RowState o{p.x, p.y, p.z, a.pi[base + c]};
      row_merge(st, o);
    }
#pragma unroll
    for (int mask = 1; mask < 64; mask <<= 1) {
      RowState o{shfl_xor(st.m, mask), shfl_xor(st.s, mask), shfl_xor(st.key, mask),
                 shfl_xor(st.idx, mask)};
      row_merge(st, o);
    }
    if (lane == 0) {
      s_lt[k - 1] = (st.m + fast_log2(st.s)) * kLn2;   // ln sum exp(t / T)
      s_star[k - 1] = st.idx;
    }
  }
  __syncthreads();
  if (lane != 0) return;
  const uint32_t req = a.req ? a.req[b] : (uint32_t)b;
  int32_t* out = a.out_tokens + (int64_t)b * (a.gamma + 1);
  int final_tok = -1;
  int resid = 0;
  bool rejected = false;
  int k = start;
  for (; k <= min(kb, a.hi); ++k) {
    int x = a.tokens[(int64_t)b * a.gamma + k - 1];
    if ((unsigned)x >= (unsigned)a.V) {
      atomicOr(a.err, kErrToken);
      x = 0;
    }
    if (a.greedy) {
      if (x == s_star[k - 1]) {
        out[A++] = x;
        continue;
      }
      final_tok = s_star[k - 1];
      rejected = true;
      break;
    }
    const float tx = a.T[(int64_t)b * a.tsb + (int64_t)(k - 1) * a.tsk + x];
    const float lpt = tx * a.invT - s_lt[k - 1];
    const int64_t o = (int64_t)b * a.gamma + k - 1;
    const float lpd = a.ytok[o] - a.lse[o];
    const float rho = fast_exp2((lpt - lpd) * kLog2e);
    const uint64_t key = stream_key(a.seed, req, (uint32_t)k, kAccept);
    const float u = hash_uniform(elem_hash((uint32_t)key, (uint32_t)(key >> 32), 0u));
    if (u < rho) {
      out[A++] = x;
      continue;
    }
    resid = k;
    rejected = true;
    break;
  }
  if (!rejected) {
    if (kb + 1 > a.hi) {            // rows left: wait for the next window
      a.vstate[b] = make_int2(A, k);
      return;
    }
    final_tok = s_star[kb];         // all kept: bonus from row K_b + 1
  }
  if (resid == 0) {
    if ((unsigned)final_tok >= (unsigned)a.V) {
      atomicOr(a.err, kErrToken);
      final_tok = 0;
    }
    out[A] = final_tok;
  }
  for (int i = A + 1; i <= a.gamma; ++i) out[i] = -1;
  a.accept_len[b] = A;
  a.resid_k[b] = resid;
  a.resid_lt[b] = resid ? s_lt[resid - 1] : 0.f;
  a.vstate[b] = make_int2(A, 0);
}

}  // namespace

const void* verify_rows_kernel() { return (const void*)&verify_rows_impl; }
const void* verify_decide_kernel() { return (const void*)&verify_decide_impl; }

}  // namespace dspark
