// Verification: per window of rows, a streaming pass over the target rows
// (one partial per 32 KB chunk), then one wave per request that merges its
// rows and takes its accept decisions.  Rows are taken in windows: a row
// after a request's first rejection is never needed, so a later window only
// reads rows of requests that have accepted every position so far (listed
// by the previous window's decisions).
//
// [blog] "形式化定义": the target scores every drafted position in one pass,
// positions are checked in order, the first rejected one is replaced by a
// target token and the rest dropped, so the output law is the target's.
// Row statistics (log-sum-exp of t/T; greedy arg-max; the bonus row's
// Gumbel-max draw from exp(t/T)) need the whole vocabulary and are formed here; the accept tests need
// only t at the drafted token, read directly by the decision kernel.  The
// residual draw at the first rejection reuses the MFMA sweep (sweep.hip).
#include "common.hpp"
#include "internal.hpp"

namespace dspark {
namespace {

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

__device__ __forceinline__ void wave_row_reduce(RowState& st) {
#pragma unroll
  for (int mask = 1; mask < 64; mask <<= 1) {
    RowState o{shfl_xor(st.m, mask), shfl_xor(st.s, mask), shfl_xor(st.key, mask), shfl_xor(st.idx, mask)};
    row_merge(st, o);
  }
}

// Leader of a thread's Gumbel-max draw over its part of a chunk: weight
// relative to 2^m, E = -log2 u, index.
struct RowLead {
  float wb, eb;
  int idx;
};

// KEYMODE 0: no key, 1: arg-max of t, 2: Gumbel-max draw from exp(t/T)
// (common.hpp; entries visited in increasing index, the leader's weight
// rescaled with the running max).
template <int KEYMODE>
__device__ __forceinline__ void row_fold(RowState& st, RowLead& ld, const float4 x, int v0, float s2, uint32_t klo,
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
  const float resc = fast_exp2(st.m - mn);
  st.s = st.s * resc + S;
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
    ld.wb *= resc;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float E = gumbel_e(klo, khi, (uint32_t)(v0 + i));
      const bool lead = e[i] * ld.eb > E * ld.wb;
      ld.wb = lead ? e[i] : ld.wb;
      ld.eb = lead ? E : ld.eb;
      ld.idx = lead ? v0 + i : ld.idx;
    }
  }
}

// One chunk of kRowsPer float4 per thread: every load is issued before the
// first is used; float4 indices at or past c1 are skipped.  A Gumbel-max
// leader becomes the key log2 w_b + m - log2 E_b at the end.
template <int KEYMODE>
__device__ __forceinline__ void row_chunk(RowState& st, const float4* p, int c0, int c1, float s2, uint32_t klo,
                                          uint32_t khi) {
  float4 x[kRowsPer];
#pragma unroll
  for (int i = 0; i < kRowsPer; ++i) x[i] = p[min(c0 + (int)threadIdx.x + i * kRowsThreads, c1 - 1)];
  RowLead ld{0.0f, 1.0f, 0x7fffffff};
#pragma unroll
  for (int i = 0; i < kRowsPer; ++i) {
    const int c = c0 + (int)threadIdx.x + i * kRowsThreads;
    if (c < c1) row_fold<KEYMODE>(st, ld, x[i], 4 * c, s2, klo, khi);
  }
  if constexpr (KEYMODE == 2) {
    if (ld.wb > 0.0f) {
      st.key = fast_log2(ld.wb) + st.m - fast_log2(ld.eb);
      st.idx = ld.idx;
    }
  }
}

// Stores and loads of the values one workgroup hands to another within a
// launch (chunk partials, request states): agent-scope atomics, which the
// other XCDs' caches cannot hold stale.
__device__ __forceinline__ void st_u32(void* p, uint32_t v) {
  __hip_atomic_store(static_cast<uint32_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_u32(const void* p) {
  return __hip_atomic_load(static_cast<const uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_state(int2* p, int2 v) {
  __hip_atomic_store(reinterpret_cast<unsigned long long*>(p),
                     (unsigned long long)(uint32_t)v.x | ((unsigned long long)(uint32_t)v.y << 32), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int2 ld_state(const int2* p) {
  const unsigned long long v =
      __hip_atomic_load(reinterpret_cast<const unsigned long long*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return make_int2((int)(uint32_t)v, (int)(uint32_t)(v >> 32));
}

// The partial (max, sum, key, index) of one 32 KB chunk of target row
// (b, k), from the whole workgroup.  Rows past K_b + 1 are skipped (the
// condition is uniform over the workgroup).
__device__ __forceinline__ void row_task(const VerifyArgs& a, int b, int k, int chunk, RowState* red) {
  const int kb = clamp_k(a.K, b, a.gamma, a.err, a.first && chunk == 0 && k == 1 && threadIdx.x == 0);
  if (k > kb + 1) return;
  const int64_t row = (int64_t)b * (a.gamma + 1) + (k - 1);
  const bool bonus = (k == kb + 1);
  const float4* p =
      reinterpret_cast<const float4*>(a.T + target_row(a.toffs, a.t_rows, a.tsb, a.tsk, b, k, a.err));
  const int nv4 = a.V >> 2;
  const int c0 = chunk * kRowsThreads * kRowsPer;
  const int c1 = min(nv4, c0 + kRowsThreads * kRowsPer);
  RowState st{-INFINITY, 0.f, -INFINITY, 0x7fffffff};
  if (a.greedy) {
    row_chunk<1>(st, p, c0, c1, a.s2, 0, 0);
  } else if (bonus) {
    const uint32_t req = a.req ? a.req[b] : (uint32_t)b;
    const uint64_t key = stream_key(a.seed, req, (uint32_t)k, kBonus);
    row_chunk<2>(st, p, c0, c1, a.s2, (uint32_t)key, (uint32_t)(key >> 32));
  } else {
    row_chunk<0>(st, p, c0, c1, a.s2, 0, 0);
  }
  // wave reduction, then across the four waves in a fixed order
  wave_row_reduce(st);
  const int wid = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wid] = st;
  __syncthreads();
  if (threadIdx.x == 0) {
    RowState acc = red[0];
#pragma unroll
    for (int w = 1; w < kRowsThreads / 64; ++w) row_merge(acc, red[w]);
    const int64_t o = row * a.n_chunks + chunk;
    if (a.decide) {
      // read within this launch by the request's decider
      st_u32(&a.pf[o].x, __float_as_uint(acc.m));
      st_u32(&a.pf[o].y, __float_as_uint(acc.s));
      st_u32(&a.pf[o].z, __float_as_uint(acc.key));
      st_u32(&a.pi[o], (uint32_t)acc.idx);
    } else {
      a.pf[o] = make_float4(acc.m, acc.s, acc.key, 0.f);
      a.pi[o] = acc.idx;
    }
  }
  __syncthreads();                                       // red is reused by the next task
}

// One wave per request: merge the chunk partials of its rows lo .. last of
// this window (8 lanes per row, 8 rows at a time), then test the rows in
// parallel (lane i tests row lo + i: the tests of different rows are
// independent, and the first rejection ends the request).  Writes the kept
// drafts, the compensation / bonus token when it is known here, the residual
// request otherwise; a request that kept every row of the window and has
// rows left stays pending for the next window.
//
// kCoherent: called inside the row pass (the partials and the request states
// of this window were written by other workgroups of the same launch).
template <bool kCoherent>
__device__ __forceinline__ void decide_request(const VerifyArgs& a, int b, int lane) {
  const int2 vs0 = a.first ? make_int2(0, 0) : a.vstate[b];   // written by the previous window
  const int kb = clamp_k(a.K, b, a.gamma, a.err, false);
  const int A0 = vs0.x;
  const int last = min(a.hi, kb + 1);
  const int n_rows = last - a.lo + 1;                      // >= 1 for a pending request
  const int n_test = max(0, min(last, kb) - a.lo + 1);     // rows with an accept test
  const int64_t row0 = (int64_t)b * (a.gamma + 1) + (a.lo - 1);
  const uint32_t req = a.req ? a.req[b] : (uint32_t)b;

  // draft-side values of the tested row of this lane (independent of the merge)
  const int k = a.lo + lane;
  int x = 0;
  float tx = 0.f, lpd = 0.f;
  if (lane < n_test) {
    x = a.tokens[(int64_t)b * a.gamma + k - 1];
    if ((unsigned)x >= (unsigned)a.V) {
      atomicOr(a.err, kErrToken);
      x = 0;
    }
    if (!a.greedy) {
      tx = a.T[target_row(a.toffs, a.t_rows, a.tsb, a.tsk, b, k, a.err) + x];
      const int64_t o = (int64_t)b * a.gamma + k - 1;
      lpd = a.ytok[o] - a.lse[o];
    }
  }
  // row statistics: lanes 8r .. 8r+7 merge row r of each group of 8 rows
  float my_lse = 0.f;   // of row lo + lane, for lane < n_rows
  int my_star = 0;
  for (int g0 = 0; g0 < n_rows; g0 += 8) {
    const int r = g0 + (lane >> 3);
    RowState st{-INFINITY, 0.f, -INFINITY, 0x7fffffff};
    if (r < n_rows) {
      const int64_t base = (row0 + r) * a.n_chunks;
      for (int c = lane & 7; c < a.n_chunks; c += 8) {
        if constexpr (kCoherent) {
          const float4* q = &a.pf[base + c];
          row_merge(st, RowState{__uint_as_float(ld_u32(&q->x)), __uint_as_float(ld_u32(&q->y)),
                                 __uint_as_float(ld_u32(&q->z)), (int)ld_u32(&a.pi[base + c])});
        } else {
          const float4 q = a.pf[base + c];
          row_merge(st, RowState{q.x, q.y, q.z, a.pi[base + c]});
        }
      }
    }
#pragma unroll
    for (int mask = 1; mask < 8; mask <<= 1) {
      RowState o{shfl_xor(st.m, mask), shfl_xor(st.s, mask), shfl_xor(st.key, mask), shfl_xor(st.idx, mask)};
      row_merge(st, o);
    }
    const float lse_r = (st.m + fast_log2(st.s)) * kLn2;   // ln sum exp(t / T)
    // lane g0 + i takes the statistics of row g0 + i (held by lane 8 i)
    const int src = ((lane - g0) & 7) * 8;
    const float l2 = __shfl(lse_r, src, 64);
    const int s2 = __shfl(st.idx, src, 64);
    if (lane >= g0 && lane < g0 + 8) {
      my_lse = l2;
      my_star = s2;
    }
  }
  bool rej = false;
  if (lane < n_test) {
    if (a.greedy) {
      rej = x != my_star;
    } else {
      const float lpt = tx * a.invT - my_lse;
      const float rho = fast_exp2((lpt - lpd) * kLog2e);
      const uint64_t key = stream_key(a.seed, req, (uint32_t)k, kAccept);
      const float u = hash_uniform(elem_hash((uint32_t)key, (uint32_t)(key >> 32), 0u));
      rej = !(u < rho);
    }
  }
  const uint64_t rmask = __ballot(rej);
  const int f = rmask ? __builtin_ctzll(rmask) : -1;       // first rejecting lane
  const int n_acc = f >= 0 ? f : n_test;
  int32_t* out = a.out_tokens + (int64_t)b * (a.gamma + 1);
  if (lane < n_acc) out[A0 + lane] = x;
  const int A = A0 + n_acc;
  int final_tok = -1;
  int resid = 0;
  float resid_lt = 0.f;
  if (f >= 0) {
    if (a.greedy)
      final_tok = __shfl(my_star, f, 64);
    else {
      resid = a.lo + f;
      resid_lt = __shfl(my_lse, f, 64);
    }
  } else if (kb + 1 <= a.hi) {
    final_tok = __shfl(my_star, kb + 1 - a.lo, 64);        // every draft kept: bonus from row K_b + 1
  } else {
    if (lane == 0) {
      if constexpr (kCoherent) {
        st_state(&a.vstate[b], make_int2(A, a.hi + 1));    // rows left: wait for the next window
      } else {
        a.vstate[b] = make_int2(A, a.hi + 1);
        if (a.list_out) a.list_out[1 + atomicAdd(a.list_out, 1)] = b;
      }
    }
    return;
  }
  for (int i = A + 1 + lane; i <= a.gamma; i += 64) out[i] = -1;
  if (lane == 0) {
    if (resid == 0) {
      if ((unsigned)final_tok >= (unsigned)a.V) {
        atomicOr(a.err, kErrToken);
        final_tok = 0;
      }
      out[A] = final_tok;
    }
    a.accept_len[b] = A;
    a.resid_k[b] = resid;
    a.resid_lt[b] = resid_lt;
    if constexpr (kCoherent)
      st_state(&a.vstate[b], make_int2(A, 0));
    else
      a.vstate[b] = make_int2(A, 0);
  }
}

__global__ __launch_bounds__(64) void verify_decide_impl(const VerifyArgs a) {
  const int b = blockIdx.x;
  if (!a.first && a.vstate[b].y == 0) return;
  decide_request<false>(a, b, threadIdx.x);
}

// Row pass of one window.  Without a work list: one workgroup per (chunk,
// request, row).  With one (later windows): a fixed grid walks the tasks
// (pending request, row, chunk) of the listed requests, so the requests
// already decided cost no workgroups.
//
// With a.decide, each task then counts itself for its request (after its
// partial has been stored coherently); the request's last task merges the
// request's rows and decides it (wave 0), and the last request decided in
// the window writes the list of the requests still pending (list_out).
// Every request of the window decides once, so the counters are back at
// zero when the window ends.
__device__ __forceinline__ void count_and_decide(const VerifyArgs& a, int b, int per, int n_pend, int* sh) {
  if (threadIdx.x == 0) {
    __builtin_amdgcn_s_waitcnt(0xF70);                   // this task's partial stores have completed
    sh[0] = (int)__hip_atomic_fetch_add(&a.dcnt[b], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  const bool last_task = sh[0] == per - 1;
  __syncthreads();
  if (!last_task) return;                                // uniform over the block
  if (threadIdx.x < 64) decide_request<true>(a, b, threadIdx.x);
  if (threadIdx.x == 0) {
    __hip_atomic_store(&a.dcnt[b], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(0xF70);                   // the request's state has been stored
    sh[0] = (int)__hip_atomic_fetch_add(a.wcnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  const bool last_req = sh[0] == n_pend - 1;
  __syncthreads();
  if (!last_req) return;
  if (threadIdx.x == 0) __hip_atomic_store(a.wcnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (!a.list_out) return;
  // every request of the window is decided: list the pending ones
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  int base = 0;
  for (int b0 = 0; b0 < a.B; b0 += kRowsThreads) {
    const int bb = b0 + (int)threadIdx.x;
    const bool pend = bb < a.B && ld_state(&a.vstate[bb]).y != 0;
    const uint64_t m = __ballot(pend);
    if (lane == 0) sh[1 + wid] = __popcll(m);
    __syncthreads();
    int off = base;
    for (int w = 0; w < wid; ++w) off += sh[1 + w];
    if (pend) a.list_out[1 + off + __popcll(m & ((1ull << lane) - 1ull))] = bb;
    int tot = 0;
    for (int w = 0; w < kRowsThreads / 64; ++w) tot += sh[1 + w];
    base += tot;
    __syncthreads();
  }
  if (threadIdx.x == 0) a.list_out[0] = base;
}

__global__ __launch_bounds__(kRowsThreads) void verify_rows_impl(const VerifyArgs a) {
  __shared__ RowState red[kRowsThreads / 64];
  __shared__ int sh[1 + kRowsThreads / 64];
  const int nrows = a.hi - a.lo + 1;
  const int per = nrows * a.n_chunks;
  if (!a.decide && a.list_out && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) a.list_out[0] = 0;
  if (!a.list_in) {
    const int chunk = blockIdx.x;
    const int b = blockIdx.y / nrows;
    const int k = a.lo + blockIdx.y % nrows;
    if (!a.first && a.vstate[b].y == 0) return;   // request already decided
    row_task(a, b, k, chunk, red);
    if (a.decide) count_and_decide(a, b, per, a.B, sh);
    return;
  }
  const int n_pend = a.list_in[0];
  // no request pending: nobody decides, so the (empty) next list is written here
  if (a.decide && n_pend == 0 && a.list_out && blockIdx.x == 0 && threadIdx.x == 0) a.list_out[0] = 0;
  const int n_tasks = n_pend * per;
  for (int t = blockIdx.x; t < n_tasks; t += gridDim.x) {
    const int i = t / per;
    const int rem = t - i * per;
    const int b = a.list_in[1 + i];
    row_task(a, b, a.lo + rem / a.n_chunks, rem % a.n_chunks, red);
    if (a.decide) count_and_decide(a, b, per, n_pend, sh);
  }
}

// Diagnostic pass: the log-normaliser of every target row 1..gamma from its
// chunk partials (one wave per row).
__global__ __launch_bounds__(64) void rows_lse_impl(const VerifyArgs a) {
  const int b = blockIdx.x;
  const int k = blockIdx.y + 1;
  const int64_t base = ((int64_t)b * (a.gamma + 1) + (k - 1)) * a.n_chunks;
  RowState st{-INFINITY, 0.f, -INFINITY, 0x7fffffff};
  for (int c = threadIdx.x; c < a.n_chunks; c += 64) {
    const float4 q = a.pf[base + c];
    row_merge(st, RowState{q.x, q.y, q.z, a.pi[base + c]});
  }
  wave_row_reduce(st);
  if (threadIdx.x == 0) a.row_lse[(int64_t)b * a.gamma + k - 1] = (st.m + fast_log2(st.s)) * kLn2;
}

}  // namespace

const void* rows_lse_kernel() { return (const void*)&rows_lse_impl; }
const void* verify_rows_kernel() { return (const void*)&verify_rows_impl; }
const void* verify_decide_kernel() { return (const void*)&verify_decide_impl; }

}  // namespace dspark
