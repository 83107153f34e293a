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
// leader becomes the key log2 w_b + m - log2 E_b at the end.  The loads are
// non-temporal: a target row is streamed once here.
__device__ __forceinline__ void row_load(float4 (&x)[kRowsPer], const float4* p, int c0, int c1) {
#pragma unroll
  for (int i = 0; i < kRowsPer; ++i) {
    const f32x4_t v = __builtin_nontemporal_load(
        reinterpret_cast<const f32x4_t*>(p + min(c0 + (int)threadIdx.x + i * kRowsThreads, c1 - 1)));
    x[i] = make_float4(v[0], v[1], v[2], v[3]);
  }
}

template <int KEYMODE>
__device__ __forceinline__ void row_fold_all(RowState& st, const float4 (&x)[kRowsPer], int c0, int c1, float s2,
                                             uint32_t klo, uint32_t khi) {
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

template <int KEYMODE>
__device__ __forceinline__ void row_chunk(RowState& st, const float4* p, int c0, int c1, float s2, uint32_t klo,
                                          uint32_t khi) {
  float4 x[kRowsPer];
  row_load(x, p, c0, c1);
  row_fold_all<KEYMODE>(st, x, c0, c1, s2, klo, khi);
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
    a.pf[o] = make_float4(acc.m, acc.s, acc.key, 0.f);
    a.pi[o] = acc.idx;
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
        const float4 q = a.pf[base + c];
        row_merge(st, RowState{q.x, q.y, q.z, a.pi[base + c]});
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
      a.vstate[b] = make_int2(A, a.hi + 1);              // rows left: wait for the next window
      if (a.list_out) a.list_out[1 + atomicAdd(a.list_out, 1)] = b;
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
    a.vstate[b] = make_int2(A, 0);
  }
}

__global__ __launch_bounds__(64) void verify_decide_impl(const VerifyArgs a) {
  const int b = blockIdx.x;
  if (!a.first && a.vstate[b].y == 0) return;
  decide_request(a, b, threadIdx.x);
}

// Row pass of one window.  Without a work list: one workgroup per (chunk,
// request, row).  With one (later windows): a fixed grid walks the tasks
// (pending request, row, chunk) of the listed requests, so the requests
// already decided cost no workgroups.
__global__ __launch_bounds__(kRowsThreads) void verify_rows_impl(const VerifyArgs a) {
  __shared__ RowState red[kRowsThreads / 64];
  const int nrows = a.hi - a.lo + 1;
  const int per = nrows * a.n_chunks;
  if (a.list_out && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) a.list_out[0] = 0;
  if (!a.list_in) {
    const int chunk = blockIdx.x;
    const int b = blockIdx.y / nrows;
    const int k = a.lo + blockIdx.y % nrows;
    if (!a.first && a.vstate[b].y == 0) return;   // request already decided
    row_task(a, b, k, chunk, red);
    return;
  }
  const int n_tasks = a.list_in[0] * per;
  for (int t = blockIdx.x; t < n_tasks; t += gridDim.x) {
    const int i = t / per;
    const int rem = t - i * per;
    const int b = a.list_in[1 + i];
    row_task(a, b, a.lo + rem / a.n_chunks, rem % a.n_chunks, red);
  }
}

// Verify chain: every needed target row in one launch, each request's rows
// read one after another and decided as soon as its row is complete, so no
// row after a request's first rejection is read and no launch separates the
// rows.  The requests are split into n_part partitions (b mod n_part), each
// served by the workgroups w with w mod n_part = p (same-address atomics are
// served one after another, so each partition keeps its own counters).  A
// partition's work items are (row, 32 KB chunk) tasks claimed from its
// ticket counter: first the chunks of row 1 of each of its requests, then
// the chunks of the rows its deciders append to its row queue.  A task's
// partial is stored coherently and counted on its row's counter; the task
// that completes a row merges the row's partials (in the order the window
// path's decision uses) and takes the row's decision: an accepted draft
// appends the next row to the queue; a rejection, or the bonus row K_b + 1,
// ends the request.  A workgroup finishes its task before it waits on the
// next ticket's row, and rows are appended by running workgroups only, so
// the launch never depends on how many of its workgroups are resident.  When
// a partition's last request is decided, its ticket counter is marked
// closed and every row slot a claimed ticket may wait on is filled with a
// closing code; the last workgroup to exit leaves the counter block at zero
// for the next launch.  Every wait is bounded (it raises the barrier error
// bit, and the workgroup then leaves).
constexpr unsigned kVqClosed = 0x80000000u;
constexpr unsigned kVqAbandon = 0x10000u;                  // row counter: its request has ended
constexpr unsigned kVqSpinLimit = 1u << 20;

__device__ __forceinline__ unsigned vq_add(unsigned* p, unsigned v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned vq_ld(const unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void vq_st(unsigned* p, unsigned v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One task of the verify chain: the partial (max, sum, key, index) of one
// 32 KB chunk of target row (b, k), as the window pass forms it, plus the
// target logit at the drafted token x_k when this chunk holds it (slot w of
// the partial; the decision needs it).  The chunk's loads go out before
// anything else is read, so the request's length K_b and the token only
// decide how the loaded values are folded.
__device__ __forceinline__ void chain_task(const VerifyArgs& a, int b, int k, int chunk, RowState* red,
                                           float* s_tx) {
  const float4* p =
      reinterpret_cast<const float4*>(a.T + target_row(a.toffs, a.t_rows, a.tsb, a.tsk, b, k, a.err));
  const int nv4 = a.V >> 2;
  const int c0 = chunk * kRowsThreads * kRowsPer;
  const int c1 = min(nv4, c0 + kRowsThreads * kRowsPer);
  float4 x[kRowsPer];
  row_load(x, p, c0, c1);
  const int kb = clamp_k(a.K, b, a.gamma, a.err, k == 1 && chunk == 0 && threadIdx.x == 0);
  int xt = -1;                                             // token tested at this row, if any
  if (!a.greedy && k <= kb) {
    xt = a.tokens[(int64_t)b * a.gamma + k - 1];
    if ((unsigned)xt >= (unsigned)a.V) xt = 0;             // the decision reports it and tests x = 0
  }
  RowState st{-INFINITY, 0.f, -INFINITY, 0x7fffffff};
  if (a.greedy) {
    row_fold_all<1>(st, x, c0, c1, a.s2, 0, 0);
  } else if (k == kb + 1) {
    const uint32_t req = a.req ? a.req[b] : (uint32_t)b;
    const uint64_t key = stream_key(a.seed, req, (uint32_t)k, kBonus);
    row_fold_all<2>(st, x, c0, c1, a.s2, (uint32_t)key, (uint32_t)(key >> 32));
  } else {
    row_fold_all<0>(st, x, c0, c1, a.s2, 0, 0);
  }
  if (xt >= 0) {
    // the thread holding float4 xt / 4 (compile-time register indices only:
    // a computed index would move x to scratch memory)
    const int c = xt >> 2;
    const int e = xt & 3;
#pragma unroll
    for (int i = 0; i < kRowsPer; ++i) {
      if (c < c1 && c == c0 + (int)threadIdx.x + i * kRowsThreads)
        *s_tx = e == 0 ? x[i].x : e == 1 ? x[i].y : e == 2 ? x[i].z : x[i].w;
    }
  }
  wave_row_reduce(st);
  const int wid = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wid] = st;
  __syncthreads();
  if (threadIdx.x == 0) {
    RowState acc = red[0];
#pragma unroll
    for (int w = 1; w < kRowsThreads / 64; ++w) row_merge(acc, red[w]);
    const int64_t o = ((int64_t)b * (a.gamma + 1) + (k - 1)) * a.n_chunks + chunk;
    st_u32(&a.pf[o].x, __float_as_uint(acc.m));
    st_u32(&a.pf[o].y, __float_as_uint(acc.s));
    st_u32(&a.pf[o].z, __float_as_uint(acc.key));
    st_u32(&a.pf[o].w, __float_as_uint(*s_tx));
    st_u32(&a.pi[o], (uint32_t)acc.idx);
  }
  __syncthreads();                                       // red and s_tx are reused by the next task
}

__device__ __forceinline__ unsigned* row_ctr(const VerifyArgs& a, int b, int k) {
  return a.vq + kVqRows + (size_t)kVqRowStride * ((int64_t)b * (a.gamma + 1) + (k - 1));
}

// Appends row k of request b to the partition's row queue (one lane).
__device__ __forceinline__ void chain_enqueue(const VerifyArgs& a, unsigned* part, unsigned* qrow, int b, int k) {
  const unsigned sl = vq_add(part + 32, 1u);
  if (sl < (unsigned)a.qcap)
    vq_st(qrow + kVqSlotStride * sl, (unsigned)((int64_t)b * (a.gamma + 1) + (k - 1)) + 1u);
  else
    atomicOr(a.err, kErrBarrier);                          // cannot happen: qcap covers every row
}

// Decisions of request b from row k on (wave 0 of the workgroup that
// completed row k; n_chunks <= 64).  A kept draft k adds its share to row
// k + 1's counter; if that completes the row (its chunks were read ahead),
// row k + 1 is decided here too.  n_req: requests of the partition, n_init:
// its row-1 tasks.
__device__ void chain_decide(const VerifyArgs& a, int b, int k, int lane, unsigned* part, unsigned* qrow, int n_req,
                             unsigned n_init) {
  const int kb = clamp_k(a.K, b, a.gamma, a.err, false);
  const uint32_t req = a.req ? a.req[b] : (uint32_t)b;
  int32_t* out = a.out_tokens + (int64_t)b * (a.gamma + 1);
  for (;;) {
    // loads that do not depend on the row's statistics go out first
    const bool test = k <= kb;
    int x = 0;
    float lpd = 0.f;
    if (test) {
      x = a.tokens[(int64_t)b * a.gamma + k - 1];
      if (!a.greedy) {
        const int64_t o = (int64_t)b * a.gamma + k - 1;
        lpd = a.ytok[o] - a.lse[o];
      }
    }
    const int64_t row = (int64_t)b * (a.gamma + 1) + (k - 1);
    // every chunk's partial at once: lane c loads chunk c
    float pm = -INFINITY, ps = 0.f, pk = -INFINITY, ptx = 0.f;
    int pidx = 0x7fffffff;
    if (lane < a.n_chunks) {
      const int64_t o = row * a.n_chunks + lane;
      const float4* q = &a.pf[o];
      pm = __uint_as_float(ld_u32(&q->x));
      ps = __uint_as_float(ld_u32(&q->y));
      pk = __uint_as_float(ld_u32(&q->z));
      ptx = __uint_as_float(ld_u32(&q->w));
      pidx = (int)ld_u32(&a.pi[o]);
    }
    if (lane == 0) vq_st(row_ctr(a, b, k), 0u);            // the row is complete: its counter is free
    // merged in the decision kernel's order: lane j < 8 takes chunks j, j + 8,
    // ... in turn, then a three-level butterfly
    RowState st{-INFINITY, 0.f, -INFINITY, 0x7fffffff};
    for (int c0 = 0; c0 < a.n_chunks; c0 += 8) {
      const int c = c0 + (lane & 7);
      const RowState o{__shfl(pm, c, 64), __shfl(ps, c, 64), __shfl(pk, c, 64), __shfl(pidx, c, 64)};
      if (lane < 8 && c < a.n_chunks) row_merge(st, o);
    }
#pragma unroll
    for (int mask = 1; mask < 8; mask <<= 1) {
      RowState o{shfl_xor(st.m, mask), shfl_xor(st.s, mask), shfl_xor(st.key, mask), shfl_xor(st.idx, mask)};
      row_merge(st, o);
    }
    const float lse_r = __shfl((st.m + fast_log2(st.s)) * kLn2, 0, 64);
    const int star = __shfl(st.idx, 0, 64);
    bool rej = false;
    if (test) {                                            // uniform over the wave
      if ((unsigned)x >= (unsigned)a.V) {
        if (lane == 0) atomicOr(a.err, kErrToken);
        x = 0;
      }
      if (a.greedy) {
        rej = x != star;
      } else {
        const float tx = __shfl(ptx, (x >> 2) / (kRowsThreads * kRowsPer), 64);
        const float lpt = tx * a.invT - lse_r;
        const float rho = fast_exp2((lpt - lpd) * kLog2e);
        const uint64_t key = stream_key(a.seed, req, (uint32_t)k, kAccept);
        const float u = hash_uniform(elem_hash((uint32_t)key, (uint32_t)(key >> 32), 0u));
        rej = !(u < rho);
      }
      if (!rej) {
        // draft k kept: row k + lookahead joins the queue, and row k + 1
        // (at most K_b + 1) gets its last share unless chunks are missing
        int next = 0;
        if (lane == 0) {
          out[k - 1] = x;
          if (k + a.lookahead <= kb + 1) chain_enqueue(a, part, qrow, b, k + a.lookahead);
          next = (vq_add(row_ctr(a, b, k + 1), 1u) & 0xFFFFu) == (unsigned)a.n_chunks;
        }
        if (!__shfl(next, 0, 64)) return;
        ++k;
        continue;
      }
    }
    // the request ends here: after k - 1 kept drafts (rejection) or all K_b;
    // rows read ahead of it are abandoned (whoever completes one frees it)
    const int A = rej ? k - 1 : kb;
    for (int i = A + 1 + lane; i <= a.gamma; i += 64) out[i] = -1;
    if (lane == 0) {
      const int last_ahead = min(k - 1 + a.lookahead, kb + 1);
      for (int j = k + 1; j <= last_ahead; ++j) {
        unsigned* cj = row_ctr(a, b, j);
        if ((vq_add(cj, 1u + kVqAbandon) & 0xFFFFu) == (unsigned)a.n_chunks) vq_st(cj, 0u);
      }
      int resid = 0;
      float resid_lt = 0.f;
      if (rej && !a.greedy) {
        resid = k;
        resid_lt = lse_r;
      } else {
        int tok = star;                                    // greedy correction, or the bonus draw
        if ((unsigned)tok >= (unsigned)a.V) {
          atomicOr(a.err, kErrToken);
          tok = 0;
        }
        out[A] = tok;
      }
      a.accept_len[b] = A;
      a.resid_k[b] = resid;
      a.resid_lt[b] = resid_lt;
      __builtin_amdgcn_s_waitcnt(0xF70);                   // outputs stored before the request counts
      const unsigned d = vq_add(part + 64, 1u);
      if (d == (unsigned)n_req - 1u) {
        // the partition's last request: close its tickets; every row slot a
        // ticket claimed before the close may wait on gets the closing code
        const unsigned o = __hip_atomic_fetch_or(part, kVqClosed, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const unsigned tq = vq_ld(part + 32);
        const unsigned t_end = o & ~kVqClosed;
        const unsigned hi = t_end > n_init ? (t_end - n_init + a.n_chunks - 1) / a.n_chunks : 0u;
        const unsigned lim = min(hi, (unsigned)a.qcap);
        for (unsigned sl = tq; sl < lim; ++sl) vq_st(qrow + kVqSlotStride * sl, kVqClosed);
        vq_st(part + 96, max(lim, tq));
      }
    }
    return;
  }
}

__global__ __launch_bounds__(kRowsThreads) void verify_chain_impl(const VerifyArgs a) {
  __shared__ RowState red[kRowsThreads / 64];
  __shared__ unsigned sh[4];
  __shared__ float s_tx;
  const int np = a.n_part;
  const int p = blockIdx.x % np;
  const int n_req = (a.B - p + np - 1) / np;               // requests p, p + np, ...
  const unsigned n_init = (unsigned)n_req * a.n_chunks;
  const int rows = a.B * (a.gamma + 1);
  unsigned* const part = a.vq + kVqPartWords * p;          // [0] tickets, [32] tail, [64] decided, [96] slots used
  unsigned* const qrow = a.vq + kVqRows + (size_t)kVqRowStride * rows + (size_t)kVqSlotStride * p * a.qcap;
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;

  if (threadIdx.x == 0) sh[0] = vq_add(part, 1u);
  __syncthreads();
  unsigned t = sh[0];
  __syncthreads();
  while (!(t & kVqClosed)) {                               // uniform over the block
    int b, k, chunk;
    if (t < n_init) {
      b = p + np * (int)(t / a.n_chunks);
      k = 1;
      chunk = (int)(t % a.n_chunks);
    } else {
      const unsigned sl = (t - n_init) / a.n_chunks;
      chunk = (int)((t - n_init) % a.n_chunks);
      if (threadIdx.x == 0) {
        unsigned code = 0;
        if (sl < (unsigned)a.qcap) {
          const unsigned limit = a.bar_test ? 64u : kVqSpinLimit;
          unsigned spins = 0;
          while ((code = a.bar_test ? 0u : vq_ld(qrow + kVqSlotStride * sl)) == 0u) {
            __builtin_amdgcn_s_sleep(2);
            if (++spins > limit) break;
          }
        }
        if (code == 0u) {                                  // gave up (or an impossible slot)
          atomicOr(a.err, kErrBarrier);
          vq_st(a.vq + kVqAbort, 1u);
          code = kVqClosed;
        }
        sh[1] = code;
      }
      __syncthreads();
      const unsigned code = sh[1];
      __syncthreads();
      if (code == kVqClosed) break;
      const int r = (int)(code - 1u);
      b = r / (a.gamma + 1);
      k = r - b * (a.gamma + 1) + 1;
    }
    // the next ticket, claimed while this task streams
    unsigned nxt = 0;
    if (threadIdx.x == 0) {
      nxt = vq_add(part, 1u);
      if (k == 1 && chunk == 0) {
        // rows 2 .. lookahead of the request are read ahead from the start
        const int kb = clamp_k(a.K, b, a.gamma, a.err, false);
        for (int j = 2; j <= min(a.lookahead, kb + 1); ++j) chain_enqueue(a, part, qrow, b, j);
      }
    }
    chain_task(a, b, k, chunk, red, &s_tx);
    if (threadIdx.x == 0) {
      __builtin_amdgcn_s_waitcnt(0xF70);                   // this task's partial is stored
      // a row is complete with its chunks and, after row 1, the previous
      // row's share (kept: decide it; abandoned: free its counter)
      unsigned* ctr = row_ctr(a, b, k);
      const unsigned old = vq_add(ctr, 1u);
      const unsigned last = (unsigned)a.n_chunks - (k > 1 ? 0u : 1u);
      const bool complete = (old & 0xFFFFu) == last;
      if (complete && (old & kVqAbandon)) vq_st(ctr, 0u);
      sh[2] = complete && !(old & kVqAbandon);
      sh[0] = nxt;
    }
    __syncthreads();
    if (sh[2] && wid == 0) chain_decide(a, b, k, lane, part, qrow, n_req, n_init);
    t = sh[0];
    __syncthreads();
  }
  // leave; the last workgroup out clears what the launch used
  if (threadIdx.x == 0) {
    __builtin_amdgcn_s_waitcnt(0xF70);
    sh[3] = vq_add(a.vq + kVqExit, 1u) == gridDim.x - 1u;
  }
  __syncthreads();
  if (!sh[3]) return;
  const bool aborted = vq_ld(a.vq + kVqAbort) != 0u;
  for (int q = 0; q < np; ++q) {
    unsigned* pq = a.vq + kVqPartWords * q;
    unsigned* rq = a.vq + kVqRows + (size_t)kVqRowStride * rows + (size_t)kVqSlotStride * q * a.qcap;
    const unsigned used = aborted ? (unsigned)a.qcap : max(vq_ld(pq + 96), vq_ld(pq + 32));
    for (unsigned sl = threadIdx.x; sl < used && sl < (unsigned)a.qcap; sl += kRowsThreads)
      vq_st(rq + kVqSlotStride * sl, 0u);
  }
  // rows read ahead of a request's end whose tickets were never claimed keep
  // a count: every row counter is cleared here
  for (int r = threadIdx.x; r < rows; r += kRowsThreads) vq_st(a.vq + kVqRows + kVqRowStride * r, 0u);
  __syncthreads();
  if (threadIdx.x < np) {
    unsigned* pq = a.vq + kVqPartWords * threadIdx.x;
    vq_st(pq, 0u);
    vq_st(pq + 32, 0u);
    vq_st(pq + 64, 0u);
    vq_st(pq + 96, 0u);
  }
  if (threadIdx.x == 0) {
    vq_st(a.vq + kVqAbort, 0u);
    vq_st(a.vq + kVqExit, 0u);
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
const void* verify_chain_kernel() { return (const void*)&verify_chain_impl; }

}  // namespace dspark
