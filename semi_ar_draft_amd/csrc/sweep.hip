// Vocabulary sweeps that carry the Markov-head bias (MFMA), for the draft
// positions and for the verify residual draw.
//
// [blog] "Markov Head：一阶转移偏置": B_k(v) = W1[x_{k-1}] . W2[:, v] with
// W1 in R^{V x r}, W2 in R^{r x V}; [teardown] "DSpark 的解法" writes it as
// B (A e_{t-1}) added to the parallel logits.  For a block of 16 vocabulary
// entries and 16 requests this is a 16 x 16 x r product: A = W2 columns (the
// [V][r] storage makes each column contiguous), B = the gathered W1 rows.
//
// Each wave owns 32 request rows and a contiguous range of 16-wide vocabulary
// tiles.  The gathered W1 rows stay in registers for the whole range; per
// tile the wave loads the W2 tile (16 x r) and the U tile (32 x 16), runs
// r/32 bf16 MFMAs per 16-row block, and folds z = U + bias into per-lane
// running statistics:
//   draft:    online log-sum-exp of y = z / T (base 2), arg-max of z
//             (greedy) or of the Gumbel key (sampling);
//   residual: arg-max of ln max(0, p_t - p_d) + Gumbel (and of the target's
//             own Gumbel key as the empty-residual fallback).
// With the 16x16x32 MFMA lane l holds rows D[4*(l/16) + i][l % 16]: four
// consecutive vocabulary entries of one request, so U is read with one
// 16-byte load per lane and the per-lane statistics need no cross-lane work
// until the end of the range.
#include "common.hpp"
#include "internal.hpp"

namespace dspark {
namespace {

// MFMA fragment traits: bf16 weights use 16x16x32 (8 values per lane per K
// step), fp32 weights 16x16x4 (1 value per lane per K step).  In both the
// K index of a lane's element is the same for the A and B operands.
template <typename WT, int R>
struct Frag;

template <int R>
struct Frag<uint16_t, R> {
  static constexpr int NS = R / 32;
  typedef bf16x8_t T;
  static __device__ __forceinline__ T load(const uint16_t* row, int s, int q) {
    return load_bf16x8(row + 32 * s + 8 * q);
  }
  static __device__ __forceinline__ T zero() { return zero_bf16x8(); }
  static __device__ __forceinline__ f32x4_t mma(T a, T b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

template <int R>
struct Frag<float, R> {
  static constexpr int NS = R / 4;
  typedef float T;
  static __device__ __forceinline__ T load(const float* row, int s, int q) { return row[4 * s + q]; }
  static __device__ __forceinline__ T zero() { return 0.0f; }
  static __device__ __forceinline__ f32x4_t mma(T a, T b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

struct LaneState {
  float m, s;       // log-sum-exp state (draft)
  float key;        // best key
  int idx;          // its vocabulary index
  float zb;         // z at the best key (sampling draft)
  float fkey;       // residual: fallback key (target Gumbel)
  int fidx;
};

__device__ __forceinline__ void lane_init(LaneState& st) {
  st.m = -INFINITY;
  st.s = 0.0f;
  st.key = -INFINITY;
  st.idx = 0x7fffffff;
  st.zb = 0.0f;
  st.fkey = -INFINITY;
  st.fidx = 0x7fffffff;
}

// Fold four z values (vocabulary v0..v0+3 of one request) into the state.
template <int MODE>
__device__ __forceinline__ void epilogue(LaneState& st, const float4 u, const f32x4_t acc,
                                         const float4 t, int v0, uint32_t klo, uint32_t khi,
                                         float invT, float s2, float ld, float lt) {
  const float z[4] = {u.x + acc[0], u.y + acc[1], u.z + acc[2], u.w + acc[3]};
  if constexpr (MODE == kModeDraftGreedy || MODE == kModeDraftSample) {
    float y2[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) y2[i] = z[i] * s2;
    const float mt = fmaxf(fmaxf(y2[0], y2[1]), fmaxf(y2[2], y2[3]));
    const float mn = fmaxf(st.m, mt);
    float acc_s = st.s * fast_exp2(st.m - mn);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc_s += fast_exp2(y2[i] - mn);
    st.s = acc_s;
    st.m = mn;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float key;
      if constexpr (MODE == kModeDraftGreedy) {
        key = z[i];
      } else {
        const float uu = hash_uniform(elem_hash(klo, khi, (uint32_t)(v0 + i)));
        key = y2[i] - gumbel_log2_term(uu);
      }
      if (key > st.key) {
        st.key = key;
        st.idx = v0 + i;
        st.zb = z[i];
      }
    }
  } else {
    const float tv[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float lpd = __builtin_fmaf(z[i], invT, -ld);    // ln p_d(v)
      const float lpt = __builtin_fmaf(tv[i], invT, -lt);   // ln p_t(v)
      const float r = fast_exp2(lpt * kLog2e) - fast_exp2(lpd * kLog2e);
      const float uu = hash_uniform(elem_hash(klo, khi, (uint32_t)(v0 + i)));
      const float gl = gumbel_log2_term(uu);
      const float key = (r > 0.0f) ? fast_log2(r) - gl : -INFINITY;
      if (key > st.key) {
        st.key = key;
        st.idx = v0 + i;
      }
      const float fkey = __builtin_fmaf(lpt, kLog2e, -gl);
      if (fkey > st.fkey) {
        st.fkey = fkey;
        st.fidx = v0 + i;
      }
    }
  }
}

template <int MODE>
__device__ __forceinline__ void lane_merge(LaneState& st, int mask) {
  if constexpr (MODE != kModeResidual) {
    const float m2 = shfl_xor(st.m, mask);
    const float s2 = shfl_xor(st.s, mask);
    softmax_merge(st.m, st.s, m2, s2);
  }
  const float k2 = shfl_xor(st.key, mask);
  const int i2 = shfl_xor(st.idx, mask);
  const float z2 = shfl_xor(st.zb, mask);
  if (key_beats(k2, i2, st.key, st.idx)) {
    st.key = k2;
    st.idx = i2;
    st.zb = z2;
  }
  if constexpr (MODE == kModeResidual) {
    const float f2 = shfl_xor(st.fkey, mask);
    const int j2 = shfl_xor(st.fidx, mask);
    if (key_beats(f2, j2, st.fkey, st.fidx)) {
      st.fkey = f2;
      st.fidx = j2;
    }
  }
}

// Blocks are dispatched to the 8 XCDs round robin.  Renumber them so that
// logical neighbours (which share a vocabulary chunk when a request batch
// spans several workgroups) land on the same XCD and its L2.
__device__ __forceinline__ int xcd_logical_block(int p, int n) {
  if ((n & 7) != 0) return p;
  return (p & 7) * (n >> 3) + (p >> 3);
}

template <typename WT, int R, int MODE>
__global__ __launch_bounds__(256) void sweep_kernel_impl(const SweepArgs a) {
  using F = Frag<WT, R>;
  constexpr int NS = F::NS;
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int q = lane >> 4;
  const int j = lane & 15;
  const int blk = a.xcd_remap ? xcd_logical_block(blockIdx.x, gridDim.x) : (int)blockIdx.x;
  const int gw = blk * kWavesPerBlock + wid;
  const int rg = gw % a.n_rg;
  const int vc = gw / a.n_rg;
  if (vc >= a.n_vc) return;

  bool ok[2];
  int rows[2];
  const float* urow[2];
  const float* trow[2];
  uint32_t klo[2], khi[2];
  float ld[2], lt[2];
  typename F::T H[2][NS];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int b = rg * kRowsPerWave + nb * 16 + j;
    bool v = b < a.B;
    int kk = a.k;
    if constexpr (MODE == kModeResidual) {
      kk = v ? a.resid_k[b] : 0;
      v = v && kk > 0 && kk <= a.gamma;
    }
    int prev = 0;
    urow[nb] = a.U;
    trow[nb] = a.T;
    klo[nb] = khi[nb] = 0;
    ld[nb] = lt[nb] = 0.0f;
    if (v) {
      prev = (kk == 1) ? a.anchor[b] : a.tokens[(int64_t)b * a.gamma + kk - 2];
      if ((unsigned)prev >= (unsigned)a.V) {
        atomicOr(a.err, kErrToken);
        prev = 0;
      }
      urow[nb] = a.U + (int64_t)b * a.usb + (int64_t)(kk - 1) * a.usk;
      if constexpr (MODE != kModeDraftGreedy) {
        const uint32_t req = a.req ? a.req[b] : (uint32_t)b;
        const uint64_t key =
            stream_key(a.seed, req, (uint32_t)kk, MODE == kModeResidual ? kResid : kDraft);
        klo[nb] = (uint32_t)key;
        khi[nb] = (uint32_t)(key >> 32);
      }
      if constexpr (MODE == kModeResidual) {
        trow[nb] = a.T + (int64_t)b * a.tsb + (int64_t)(kk - 1) * a.tsk;
        ld[nb] = a.lse[(int64_t)b * a.gamma + kk - 1];
        lt[nb] = a.resid_lt[b];
      }
    }
    ok[nb] = v;
    rows[nb] = b;
    const WT* w1row = static_cast<const WT*>(a.W1) + (int64_t)prev * R;
#pragma unroll
    for (int s = 0; s < NS; ++s) H[nb][s] = v ? F::load(w1row, s, q) : F::zero();
  }
  if constexpr (MODE == kModeResidual) {
    if (!__any(ok[0] || ok[1])) return;
  }

  LaneState st[2];
  lane_init(st[0]);
  lane_init(st[1]);

  const int t0 = (int)((int64_t)a.n_tiles * vc / a.n_vc);
  const int t1 = (int)((int64_t)a.n_tiles * (vc + 1) / a.n_vc);
  const WT* W2 = static_cast<const WT*>(a.W2);
  for (int t = t0; t < t1; ++t) {
    const int v0 = t * kTileV;
    const WT* w2row = W2 + (int64_t)(v0 + j) * R;
    typename F::T A[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) A[s] = F::load(w2row, s, q);
    float4 uu[2], tt[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      uu[nb] = ok[nb] ? *reinterpret_cast<const float4*>(urow[nb] + v0 + 4 * q)
                      : make_float4(0.f, 0.f, 0.f, 0.f);
      if constexpr (MODE == kModeResidual) {
        tt[nb] = ok[nb] ? *reinterpret_cast<const float4*>(trow[nb] + v0 + 4 * q)
                        : make_float4(0.f, 0.f, 0.f, 0.f);
      } else {
        tt[nb] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    f32x4_t acc[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) acc[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NS; ++s) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) acc[nb] = F::mma(A[s], H[nb][s], acc[nb]);
    }
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      if (ok[nb])
        epilogue<MODE>(st[nb], uu[nb], acc[nb], tt[nb], v0 + 4 * q, klo[nb], khi[nb], a.invT,
                       a.s2, ld[nb], lt[nb]);
    }
  }

#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    lane_merge<MODE>(st[nb], 16);
    lane_merge<MODE>(st[nb], 32);
    if (q == 0 && ok[nb]) {
      const int64_t o = (int64_t)rows[nb] * a.n_vc + vc;
      if constexpr (MODE == kModeResidual) {
        a.pf[o] = make_float4(st[nb].key, st[nb].fkey, 0.f, 0.f);
        a.pi[o] = make_int2(st[nb].idx, st[nb].fidx);
      } else {
        a.pf[o] = make_float4(st[nb].m, st[nb].s, st[nb].key, st[nb].zb);
        a.pi[o] = make_int2(st[nb].idx, 0);
      }
    }
  }
}

// One wave per request row: merge the per-chunk partials of a draft
// position, write x_k, ln-normaliser and y at x_k.
__global__ __launch_bounds__(64) void combine_draft_impl(const CombineArgs a) {
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  float m = -INFINITY, s = 0.f, key = -INFINITY, zb = 0.f;
  int idx = 0x7fffffff;
  const int64_t base = (int64_t)b * a.n_vc;
  for (int i = lane; i < a.n_vc; i += 64) {
    const float4 p = a.pf[base + i];
    const int pi = a.pi[base + i].x;
    softmax_merge(m, s, p.x, p.y);
    if (key_beats(p.z, pi, key, idx)) {
      key = p.z;
      idx = pi;
      zb = p.w;
    }
  }
#pragma unroll
  for (int mask = 1; mask < 64; mask <<= 1) {
    const float m2 = shfl_xor(m, mask), s2 = shfl_xor(s, mask);
    const float k2 = shfl_xor(key, mask), z2 = shfl_xor(zb, mask);
    const int i2 = shfl_xor(idx, mask);
    softmax_merge(m, s, m2, s2);
    if (key_beats(k2, i2, key, idx)) {
      key = k2;
      idx = i2;
      zb = z2;
    }
  }
  if (lane == 0) {
    if ((unsigned)idx >= (unsigned)a.V) {
      atomicOr(a.err, kErrToken);
      idx = 0;
    }
    const int64_t o = (int64_t)b * a.gamma + a.k - 1;
    a.tokens[o] = idx;
    a.lse[o] = (m + fast_log2(s)) * kLn2;
    a.ytok[o] = a.greedy ? key : zb * a.invT;
  }
}

// One wave per request with a pending residual draw: merge its partials and
// write the emitted token after the accepted prefix.
__global__ __launch_bounds__(64) void combine_resid_impl(const CombineArgs a) {
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  if (a.resid_k[b] <= 0) return;
  float key = -INFINITY, fkey = -INFINITY;
  int idx = 0x7fffffff, fidx = 0x7fffffff;
  const int64_t base = (int64_t)b * a.n_vc;
  for (int i = lane; i < a.n_vc; i += 64) {
    const float4 p = a.pf[base + i];
    const int2 pi = a.pi[base + i];
    if (key_beats(p.x, pi.x, key, idx)) {
      key = p.x;
      idx = pi.x;
    }
    if (key_beats(p.y, pi.y, fkey, fidx)) {
      fkey = p.y;
      fidx = pi.y;
    }
  }
#pragma unroll
  for (int mask = 1; mask < 64; mask <<= 1) {
    const float k2 = shfl_xor(key, mask), f2 = shfl_xor(fkey, mask);
    const int i2 = shfl_xor(idx, mask), j2 = shfl_xor(fidx, mask);
    if (key_beats(k2, i2, key, idx)) {
      key = k2;
      idx = i2;
    }
    if (key_beats(f2, j2, fkey, fidx)) {
      fkey = f2;
      fidx = j2;
    }
  }
  if (lane == 0) {
    int tok = (key > -INFINITY) ? idx : fidx;
    if ((unsigned)tok >= (unsigned)a.V) {
      atomicOr(a.err, kErrToken);
      tok = 0;
    }
    const int A = a.accept_len[b];
    a.out_tokens[(int64_t)b * (a.gamma + 1) + A] = tok;
  }
}

}  // namespace

const void* sweep_kernel(int wdtype, int r, int mode) {
#define DSPARK_SWEEP_CASE(WT, R)                                                        \
  if (r == R) {                                                                         \
    if (mode == kModeDraftGreedy) return (const void*)&sweep_kernel_impl<WT, R, kModeDraftGreedy>; \
    if (mode == kModeDraftSample) return (const void*)&sweep_kernel_impl<WT, R, kModeDraftSample>; \
    if (mode == kModeResidual) return (const void*)&sweep_kernel_impl<WT, R, kModeResidual>;       \
    return nullptr;                                                                     \
  }
  if (wdtype == 1) {
    DSPARK_SWEEP_CASE(uint16_t, 32)
    DSPARK_SWEEP_CASE(uint16_t, 64)
    DSPARK_SWEEP_CASE(uint16_t, 128)
    DSPARK_SWEEP_CASE(uint16_t, 256)
  } else if (wdtype == 0) {
    DSPARK_SWEEP_CASE(float, 32)
    DSPARK_SWEEP_CASE(float, 64)
    DSPARK_SWEEP_CASE(float, 128)
    DSPARK_SWEEP_CASE(float, 256)
  }
#undef DSPARK_SWEEP_CASE
  return nullptr;
}

const void* combine_draft_kernel() { return (const void*)&combine_draft_impl; }
const void* combine_resid_kernel() { return (const void*)&combine_resid_impl; }

}  // namespace dspark
