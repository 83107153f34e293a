// Vocabulary sweeps that carry the Markov-head bias (MFMA), for the draft
// positions, the verify residual draw and the acceptance-probability pass;
// and, for small batches, the whole-draft kernel that runs every position of
// a draft in one launch (draft_persist_impl, further down).
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
//             (greedy) or the Gumbel-max draw from exp(y) (sampling);
//   residual: the Gumbel-max draw from max(0, p_t - p_d) (and from p_t as
//             the empty-residual fallback).
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
  // fp32 operand as hi + lo bf16 fragments (hi = RNE(x), lo = RNE(x - hi)):
  // two MFMAs then carry x to about 2^-16 relative.
  static constexpr bool kSplit = true;
  static __device__ __forceinline__ void split(const float* row, int s, int q, T& hi, T& lo) {
    const float4 a = *reinterpret_cast<const float4*>(row + 32 * s + 8 * q);
    const float4 b = *reinterpret_cast<const float4*>(row + 32 * s + 8 * q + 4);
    const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const __bf16 h = (__bf16)v[i];
      hi[i] = h;
      lo[i] = (__bf16)(v[i] - (float)h);
    }
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
  static constexpr bool kSplit = false;   // fp32 operands are taken whole
  static __device__ __forceinline__ void split(const float* row, int s, int q, T& hi, T& lo) {
    hi = row[4 * s + q];
    lo = 0.0f;
  }
};

struct LaneState {
  float m, s;       // log-sum-exp state (draft)
  float key;        // best key
  int idx;          // its vocabulary index
  float zb;         // draft: y (tempered logit) at the best entry; greedy: z
  float fkey;       // residual: fallback key (draw from p_t)
  int fidx;
  // greedy draft, during the range: the leading group (first entry g, its
  // four z values)
  int g;
  float zg[4];
  // sampling draft and residual, during the range: the leader's weight (the
  // draft: relative to 2^m) and its E = -log2 u; residual: pb, ebf for the
  // fallback draw from p_t
  float sb, eb;
  float pb, ebf;
};

__device__ __forceinline__ void lane_init(LaneState& st) {
  st.m = -INFINITY;
  st.s = 0.0f;
  st.key = -INFINITY;
  st.idx = 0x7fffffff;
  st.zb = 0.0f;
  st.fkey = -INFINITY;
  st.fidx = 0x7fffffff;
  st.g = -1;
#pragma unroll
  for (int i = 0; i < 4; ++i) st.zg[i] = 0.0f;
  st.sb = 0.0f;
  st.eb = 1.0f;
  st.pb = 0.0f;
  st.ebf = 1.0f;
}

// Draft modes: fold the NTL tiles of one step (per lane and request row,
// NTL groups of four consecutive vocabulary entries, z = U + bias straight
// from the MFMA, whose accumulator was initialised with U) into the state:
// one max and one rescale per row and step for the online log-sum-exp, and
// the leader of the range so far, tracked without branches (with 64 lanes
// per wave some lane nearly always finds a new leader, so a branch would be
// taken on almost every step).
//
// Greedy: the group of four with the largest z (first such group on ties);
// the entry within it is resolved once, at the end of the range.
// Sampling, Gumbel-max (common.hpp): entry v with weight w_v = 2^(y2_v - m)
// (the softmax term) leads while w_v / E_v is the largest, compared as
// w_v E_b > E_v w_b with the leader's w_b rescaled together with the running
// max; entries are visited in increasing v, so equal keys keep the lower one.
template <int MODE, int NTL>
__device__ __forceinline__ void fold_draft(LaneState& st, const f32x4_t (&z)[NTL], int v0, uint32_t klo,
                                           uint32_t khi, float s2) {
  float zt[NTL];
#pragma unroll
  for (int h = 0; h < NTL; ++h) zt[h] = fmaxf(fmaxf(z[h][0], z[h][1]), fmaxf(z[h][2], z[h][3]));
  float zmax = zt[0];
#pragma unroll
  for (int h = 1; h < NTL; ++h) zmax = fmaxf(zmax, zt[h]);
  const float mn = fmaxf(st.m, zmax * s2);
  float e[NTL][4];
  float tot = 0.0f;
#pragma unroll
  for (int h = 0; h < NTL; ++h) {
#pragma unroll
    for (int i = 0; i < 4; ++i) e[h][i] = fast_exp2(__builtin_fmaf(z[h][i], s2, -mn));
    tot += (e[h][0] + e[h][1]) + (e[h][2] + e[h][3]);
  }
  const float resc = fast_exp2(st.m - mn);
  st.s = __builtin_fmaf(st.s, resc, tot);
  st.m = mn;
  if constexpr (MODE == kModeDraftGreedy) {
#pragma unroll
    for (int h = 0; h < NTL; ++h) {
      const bool lead = zt[h] > st.key;
      st.key = lead ? zt[h] : st.key;
      st.g = lead ? v0 + kTileV * h : st.g;
#pragma unroll
      for (int i = 0; i < 4; ++i) st.zg[i] = lead ? z[h][i] : st.zg[i];
    }
  } else {
    st.sb *= resc;
#pragma unroll
    for (int h = 0; h < NTL; ++h) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int v = v0 + kTileV * h + i;
        const float E = gumbel_e(klo, khi, (uint32_t)v);
        const bool lead = e[h][i] * st.eb > E * st.sb;
        st.sb = lead ? e[h][i] : st.sb;
        st.eb = lead ? E : st.eb;
        st.idx = lead ? v : st.idx;
      }
    }
  }
}

// End of a range.  Greedy: the lowest entry of the leading group holding the
// maximum.  Sampling: the leader's key log2 w_b + m - log2 E_b and its
// tempered logit y = (log2 w_b + m) ln 2.
template <int MODE>
__device__ __forceinline__ void resolve_draft(LaneState& st, uint32_t klo, uint32_t khi, float s2) {
  if constexpr (MODE == kModeDraftGreedy) {
    if (st.g < 0) return;                                // empty range
    int i = 3;
#pragma unroll
    for (int k = 2; k >= 0; --k) i = (st.zg[k] == st.key) ? k : i;
    st.idx = st.g + i;
    st.zb = st.key;
  } else {
    if (!(st.sb > 0.0f)) return;                         // empty range
    const float y2 = fast_log2(st.sb) + st.m;
    st.key = y2 - fast_log2(st.eb);
    st.zb = y2 * kLn2;
  }
}

// Residual and acceptance-probability modes: fold four values of
// z = U + bias and of the target row into the state.
template <int MODE>
__device__ __forceinline__ void epilogue(LaneState& st, const f32x4_t z, const float4 t, int v0,
                                         uint32_t klo, uint32_t khi, float invT, float ld, float lt) {
  if constexpr (MODE == kModeAlpha) {
    // acceptance probability: sum over v of min(p_t(v), p_d(v))
    const float tv[4] = {t.x, t.y, t.z, t.w};
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float pt = fast_exp2(__builtin_fmaf(tv[i], invT, -lt) * kLog2e);
      const float pd = fast_exp2(__builtin_fmaf(z[i], invT, -ld) * kLog2e);
      acc += fminf(pt, pd);
    }
    st.s += acc;
  } else {
    // residual: Gumbel-max on the weights r_v = max(0, p_t - p_d); the
    // fallback (empty residual) draws from p_t with the same uniforms.  Both
    // leaders are tracked without branches (r_v E_b > E_v r_b; the
    // probabilities need no running rescale); zero weights never lead.
    const float tv[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float pt = fast_exp2(__builtin_fmaf(tv[i], invT, -lt) * kLog2e);
      const float pd = fast_exp2(__builtin_fmaf(z[i], invT, -ld) * kLog2e);
      const float r = fmaxf(pt - pd, 0.0f);
      const int v = v0 + i;
      const float E = gumbel_e(klo, khi, (uint32_t)v);
      const bool lr = r * st.eb > E * st.sb;
      st.sb = lr ? r : st.sb;
      st.eb = lr ? E : st.eb;
      st.idx = lr ? v : st.idx;
      const bool lf = pt * st.ebf > E * st.pb;
      st.pb = lf ? pt : st.pb;
      st.ebf = lf ? E : st.ebf;
      st.fidx = lf ? v : st.fidx;
    }
  }
}

// End of a residual range: the keys log2 r_b - log2 E_b (and for p_t).
__device__ __forceinline__ void resolve_resid(LaneState& st) {
  if (st.sb > 0.0f) st.key = fast_log2(st.sb) - fast_log2(st.eb);
  if (st.pb > 0.0f) st.fkey = fast_log2(st.pb) - fast_log2(st.ebf);
}

template <int MODE>
__device__ __forceinline__ void lane_merge(LaneState& st, int mask) {
  if constexpr (MODE == kModeAlpha) {
    st.s += shfl_xor(st.s, mask);
    return;
  }
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

// Per-lane row state of one wave: the two 16-row MFMA blocks of row group rg.
// A row that is not active (past B, or no residual pending) reads request
// 0's first row so that every load is unconditional; its statistics are
// never written.
//
// HS selects the MFMA B operand (the rank-r vector the bias is projected
// from): 0 = the Markov head's W1 row of the previous token; 1 = the GRU
// head's fp32 state s_{k-1} of the request (hstate [gamma][B][r]), split
// into hi + lo bf16 fragments for bf16 weights.
template <typename WT, int R, int MODE, int HS = 0, int NBW = 2>
struct WaveRows {
  using F = Frag<WT, R>;
  using FragT = typename F::T;
  static constexpr int NS = F::NS;
  static constexpr bool kLo = HS == 1 && F::kSplit;
  static constexpr int kRows = 16 * NBW;            // request rows of the wave
  bool ok[NBW];
  int rows[NBW];
  int64_t uoff[NBW], toff[NBW];
  uint32_t klo[NBW], khi[NBW];
  float ld[NBW], lt[NBW];
  FragT H[NBW][NS];
  FragT Hlo[NBW][kLo ? NS : 1];

  int kk[NBW];

  // Row identities and stream offsets (the residual reads its position).
  __device__ __forceinline__ void setup_rows(const SweepArgs& a, int rg, int j) {
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
      const int b = rg * kRows + nb * 16 + j;
      bool v = b < a.B;
      int k = a.k;
      if constexpr (MODE == kModeResidual) {
        k = v ? a.resid_k[b] : 0;
        v = v && k > 0 && k <= a.gamma;
      }
      uoff[nb] = v ? (int64_t)b * a.usb + (int64_t)(k - 1) * a.usk : 0;
      toff[nb] = (v && (MODE == kModeResidual || MODE == kModeAlpha))
                     ? target_row(a.toffs, a.t_rows, a.tsb, a.tsk, b, k, a.err)
                     : 0;
      ok[nb] = v;
      rows[nb] = b;
      kk[nb] = k;
    }
  }

  // Previous token, its gathered W1 row (MFMA B operand), stream keys and
  // the residual's normalisers.  In the draft the previous token is the
  // maximum over the previous position's slot groups: the four lanes of a
  // row (q = 0..3) read a quarter of the groups each and share the maximum.
  // kCoherent: the previous position's slots were written by workgroups of
  // the same launch (the chained draft kernel), so they are read with
  // agent-scope atomic loads rather than through the caches.
  template <bool kCoherent = false>
  __device__ __forceinline__ void setup_rest(const SweepArgs& a, int q) {
    // loads that do not depend on the previous token go out first (the
    // error-flag atomic below would otherwise keep them behind the chain)
    uint32_t req[NBW];
    int given[NBW];                                      // anchor, or the drafted previous token
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
      const int b = rows[nb];
      const int k = kk[nb];
      req[nb] = 0u;
      given[nb] = 0;
      ld[nb] = lt[nb] = 0.0f;
      if (ok[nb]) {
        if constexpr (MODE == kModeDraftSample || MODE == kModeResidual) req[nb] = a.req ? a.req[b] : (uint32_t)b;
        if (HS == 0) {
          if (k == 1)
            given[nb] = a.anchor[b];
          else if (MODE == kModeResidual || MODE == kModeAlpha || !a.best_prev)
            given[nb] = a.tokens[(int64_t)b * a.gamma + k - 2];
        }
        if constexpr (MODE == kModeResidual) {
          ld[nb] = a.lse[(int64_t)b * a.gamma + k - 1];
          lt[nb] = a.resid_lt[b];
        }
        if constexpr (MODE == kModeAlpha) {
          ld[nb] = a.lse[(int64_t)b * a.gamma + k - 1];
          lt[nb] = a.resid_lt[(int64_t)b * a.gamma + k - 1];   // target log-normaliser of row (b, k)
        }
      }
    }
    unsigned long long pb[NBW];
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) pb[nb] = 0ull;
    if (HS == 0 && MODE != kModeResidual && MODE != kModeAlpha && a.best_prev) {
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) {
        if (ok[nb]) {
#pragma unroll
          for (int i = 0; i < kBestGroups / 4; ++i) {
            const unsigned long long* sp = a.best_prev + (int64_t)(q * (kBestGroups / 4) + i) * a.B + rows[nb];
            const unsigned long long v =
                kCoherent ? __hip_atomic_load(sp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : *sp;
            pb[nb] = v > pb[nb] ? v : pb[nb];
          }
        }
#pragma unroll
        for (int m = 16; m <= 32; m <<= 1) {
          const unsigned long long o = __shfl_xor(pb[nb], m, 64);
          pb[nb] = o > pb[nb] ? o : pb[nb];
        }
      }
    }
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
      const int b = rows[nb];
      const int k = kk[nb];
      int prev = 0;
      klo[nb] = khi[nb] = 0;
      if (ok[nb] && HS == 0) {
        if (k != 1 && MODE != kModeResidual && MODE != kModeAlpha && a.best_prev)
          prev = best_index(pb[nb]);
        else
          prev = given[nb];
        if ((unsigned)prev >= (unsigned)a.V) {
          atomicOr(a.err, kErrToken);
          prev = 0;
        }
      }
      if (ok[nb]) {
        if constexpr (MODE == kModeDraftSample || MODE == kModeResidual) {
          const uint64_t key =
              stream_key(a.seed, req[nb], (uint32_t)k, MODE == kModeResidual ? kResid : kDraft);
          klo[nb] = (uint32_t)key;
          khi[nb] = (uint32_t)(key >> 32);
        }
      }
      if constexpr (HS == 0 && sizeof(FragT) == 16) {
        // bf16: the B fragment of lane (j, q) at step s is 16 bytes of row j;
        // loaded directly, every quarter-wave would touch 16 rows.  Instead
        // lane L loads that part of row L / 4 which lane (L / 4, L % 4)
        // needs (a quarter-wave reads 4 rows x 64 contiguous bytes), and a
        // lane transpose (ds_bpermute) hands it over: lane (j, q) takes lane
        // 4 j + q's word.
        const int lane = threadIdx.x & 63;               // = 16 q + j
        const int src_prev = __shfl(prev, lane >> 2, 64);
        const WT* w1row = static_cast<const WT*>(a.W1) + (int64_t)src_prev * R;
        const int from = 4 * (4 * (lane & 15) + q);
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          union { FragT f; int w[4]; } x, y;
          x.f = F::load(w1row, s, lane & 3);
#pragma unroll
          for (int d = 0; d < 4; ++d) y.w[d] = __builtin_amdgcn_ds_bpermute(from, x.w[d]);
          H[nb][s] = y.f;
        }
      } else if constexpr (HS == 0) {
        const WT* w1row = static_cast<const WT*>(a.W1) + (int64_t)prev * R;
#pragma unroll
        for (int s = 0; s < NS; ++s) H[nb][s] = F::load(w1row, s, q);
      } else if constexpr (sizeof(FragT) == 16) {
        // state of position k (inactive rows: request 0, position 1), loaded
        // like the W1 rows above: lane L reads that part of row L / 4 which
        // lane (L / 4, L % 4) needs, splits it, and the lane transpose hands
        // over the hi and lo fragments
        const int lane = threadIdx.x & 63;
        const int srow_idx = ok[nb] ? (k - 1) * a.B + b : 0;
        const int src_row = __shfl(srow_idx, lane >> 2, 64);
        const float* srow = a.hstate + (int64_t)src_row * R;
        const int from = 4 * (4 * (lane & 15) + q);
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          union { FragT f; int w[4]; } xh, xl, yh, yl;
          F::split(srow, s, lane & 3, xh.f, xl.f);
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            yh.w[d] = __builtin_amdgcn_ds_bpermute(from, xh.w[d]);
            yl.w[d] = __builtin_amdgcn_ds_bpermute(from, xl.w[d]);
          }
          H[nb][s] = yh.f;
          Hlo[nb][kLo ? s : 0] = yl.f;
        }
      } else {
        // state of position k (inactive rows: request 0, position 1)
        const float* srow = a.hstate + ((int64_t)(ok[nb] ? k - 1 : 0) * a.B + (ok[nb] ? b : 0)) * R;
#pragma unroll
        for (int s = 0; s < NS; ++s) F::split(srow, s, q, H[nb][s], Hlo[nb][kLo ? s : 0]);
      }
    }
  }

  __device__ __forceinline__ void setup(const SweepArgs& a, int rg, int j, int q) {
    setup_rows(a, rg, j);
    setup_rest(a, q);
  }

  // z = U + bias of one tile for both blocks (U initialises the accumulators).
  __device__ __forceinline__ void mma_tile(f32x4_t (&acc)[NBW], const FragT (&A)[NS], const float4 (&uu)[NBW]) const {
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) acc[nb] = f32x4_t{uu[nb].x, uu[nb].y, uu[nb].z, uu[nb].w};
#pragma unroll
    for (int s = 0; s < NS; ++s) {
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) acc[nb] = F::mma(A[s], H[nb][s], acc[nb]);
    }
    if constexpr (kLo) {
#pragma unroll
      for (int s = 0; s < NS; ++s) {
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) acc[nb] = F::mma(A[s], Hlo[nb][s], acc[nb]);
      }
    }
  }

  // Draft modes: fold NTL consecutive tiles (acc[h][nb], tile t + h).
  template <int NTL>
  __device__ __forceinline__ void fold(const SweepArgs& a, LaneState (&st)[NBW], const f32x4_t (&acc)[NTL][NBW], int t,
                                       int q) const {
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
      f32x4_t z[NTL];
#pragma unroll
      for (int h = 0; h < NTL; ++h) z[h] = acc[h][nb];
      fold_draft<MODE, NTL>(st[nb], z, t * kTileV + 4 * q, klo[nb], khi[nb], a.s2);
    }
  }

  // One tile: z = U + bias, then fold.
  __device__ __forceinline__ void compute(const SweepArgs& a, LaneState (&st)[NBW], int t, int q,
                                          const FragT (&A)[NS], const float4 (&uu)[NBW],
                                          const float4 (&tt)[NBW]) const {
    f32x4_t acc[1][NBW];
    mma_tile(acc[0], A, uu);
    if constexpr (MODE == kModeDraftGreedy || MODE == kModeDraftSample) {
      fold<1>(a, st, acc, t, q);
    } else {
      const int vb = t * kTileV + 4 * q;
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb)
        epilogue<MODE>(st[nb], acc[0][nb], tt[nb], vb, klo[nb], khi[nb], a.invT, ld[nb], lt[nb]);
    }
  }

  __device__ __forceinline__ void finish(const SweepArgs& a, LaneState (&st)[NBW], int q, int vc) const {
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
      if constexpr (MODE == kModeDraftGreedy || MODE == kModeDraftSample)
        resolve_draft<MODE>(st[nb], klo[nb], khi[nb], a.s2);
      else if constexpr (MODE == kModeResidual)
        resolve_resid(st[nb]);
      lane_merge<MODE>(st[nb], 16);
      lane_merge<MODE>(st[nb], 32);
      if (q == 0 && ok[nb]) {
        const int64_t o = (int64_t)rows[nb] * a.n_vc + vc;
        if constexpr (MODE == kModeAlpha) {
          a.pf[o] = make_float4(st[nb].s, 0.f, 0.f, 0.f);
        } else if constexpr (MODE == kModeResidual) {
          a.pf[o] = make_float4(st[nb].key, st[nb].fkey, 0.f, 0.f);
          a.pi[o] = make_int2(st[nb].idx, st[nb].fidx);
        } else {
          a.pf[o] = make_float4(st[nb].m, st[nb].s, st[nb].key, st[nb].zb);
          a.pi[o] = make_int2(st[nb].idx, 0);
          // publish the chunk's winner into its slot group (no return value:
          // the next position reads the groups after this kernel ends)
          if (a.best) {
            unsigned long long* slot = a.best + (int64_t)(vc % kBestGroups) * a.B + rows[nb];
            __hip_atomic_fetch_max(slot, pack_best(st[nb].key, st[nb].idx), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
          }
        }
      }
    }
  }
};

// Private-tile variant: every wave owns its vocabulary chunk and loads its W2
// tiles itself (used when no two waves share a chunk, e.g. B <= 64, and for
// fp32 or narrow weights).  Double-buffered in registers.
template <typename WT, int R, int MODE, int HS>
__global__ __launch_bounds__(256) void sweep_private_impl(const SweepArgs a) {
  using WR = WaveRows<WT, R, MODE, HS>;
  using F = typename WR::F;
  using FragT = typename WR::FragT;
  constexpr int NS = WR::NS;
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int q = lane >> 4;
  const int j = lane & 15;
  const int blk = a.xcd_remap ? xcd_logical_block(blockIdx.x, gridDim.x) : (int)blockIdx.x;
  const int gw = blk * kWavesPerBlock + wid;
  const int rg = gw % a.n_rg;
  const int vc = gw / a.n_rg;
  if (vc >= a.n_vc) return;
  WR w;
  w.setup(a, rg, j, q);
  if constexpr (MODE == kModeResidual) {
    if (!__any(w.ok[0] || w.ok[1])) return;
  }
  LaneState st[2];
  lane_init(st[0]);
  lane_init(st[1]);
  const int t0 = (int)((int64_t)a.n_tiles * vc / a.n_vc);
  const int t1 = (int)((int64_t)a.n_tiles * (vc + 1) / a.n_vc);
  const WT* __restrict__ W2 = static_cast<const WT*>(a.W2);
  // bf16 weights: a direct load of the MFMA fragments (and of U) has every
  // quarter-wave touch 16 rows; instead lane L loads what lane (L / 4, L % 4)
  // needs (4 rows x 64 contiguous bytes per quarter-wave) and the lane
  // transpose (ds_bpermute) at use time hands it over, so the loads of the
  // next tile stay in flight meanwhile.
  constexpr bool kT = sizeof(FragT) == 16;
  const int src_lane = kT ? (lane >> 2) : j;
  const int src_q = kT ? (lane & 3) : q;
  const int from = 4 * (4 * j + q);
  int64_t uoff_t[2], toff_t[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    uoff_t[nb] = kT ? __shfl(w.uoff[nb], src_lane, 64) : w.uoff[nb];
    toff_t[nb] = kT ? __shfl(w.toff[nb], src_lane, 64) : w.toff[nb];
  }
  auto load_a = [&](int t, FragT (&A)[NS]) {
    const WT* w2row = W2 + (int64_t)(t * kTileV + src_lane) * R;
#pragma unroll
    for (int s = 0; s < NS; ++s) A[s] = F::load(w2row, s, src_q);
  };
  auto load_ut = [&](int t, float4 (&uu)[2], float4 (&tt)[2]) {
    const int v0 = t * kTileV + 4 * src_q;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      uu[nb] = *reinterpret_cast<const float4*>(a.U + uoff_t[nb] + v0);
      if constexpr (MODE == kModeResidual || MODE == kModeAlpha)
        tt[nb] = *reinterpret_cast<const float4*>(a.T + toff_t[nb] + v0);
      else
        tt[nb] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  auto xpose4 = [&](float4& v) {
    if constexpr (kT) {
      v.x = __int_as_float(__builtin_amdgcn_ds_bpermute(from, __float_as_int(v.x)));
      v.y = __int_as_float(__builtin_amdgcn_ds_bpermute(from, __float_as_int(v.y)));
      v.z = __int_as_float(__builtin_amdgcn_ds_bpermute(from, __float_as_int(v.z)));
      v.w = __int_as_float(__builtin_amdgcn_ds_bpermute(from, __float_as_int(v.w)));
    }
  };
  auto compute_t = [&](int t, FragT (&A)[NS], float4 (&uu)[2], float4 (&tt)[2]) {
    if constexpr (kT) {
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        union { FragT f; int w[4]; } x;
        x.f = A[s];
#pragma unroll
        for (int d = 0; d < 4; ++d) x.w[d] = __builtin_amdgcn_ds_bpermute(from, x.w[d]);
        A[s] = x.f;
      }
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        xpose4(uu[nb]);
        if constexpr (MODE == kModeResidual || MODE == kModeAlpha) xpose4(tt[nb]);
      }
    }
    w.compute(a, st, t, q, A, uu, tt);
  };
  if (t0 < t1) {
    FragT A0[NS], A1[NS];
    float4 u0[2], u1[2], x0[2], x1[2];
    load_a(t0, A0);
    load_ut(t0, u0, x0);
    for (int t = t0; t < t1; t += 2) {
      const int tn = min(t + 1, t1 - 1);
      load_a(tn, A1);
      load_ut(tn, u1, x1);
      compute_t(t, A0, u0, x0);
      if (t + 1 >= t1) break;
      const int tn2 = min(t + 2, t1 - 1);
      load_a(tn2, A0);
      load_ut(tn2, u0, x0);
      compute_t(t + 1, A1, u1, x1);
    }
  }
  w.finish(a, st, q, vc);
}

typedef __attribute__((address_space(3))) unsigned char lds_u8_t;

// Direct global->LDS load of 16 bytes per lane (global_load_lds_dwordx4):
// lane i's 16 bytes land at LDS byte address lds + 16 i; M0 carries the wave-
// uniform base and is restored afterwards.  Written as inline assembly so
// that the compiler keeps no books on it: its own wait-count tracking of such
// loads cannot tell the slots of a ring apart and would wait for every load
// in flight before each LDS read.  The kernels below order these loads
// explicitly with ring_wait_barrier; the memory clobber keeps the compiler
// from moving memory accesses across them.  kStream: a non-temporal load,
// for rows read once (U, target rows), so that they do not displace what
// the caches should keep (W2, re-read by every position, stays in the
// last-level cache).
template <bool kStream = false>
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  uint32_t saved;
  if constexpr (kStream) {
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "global_load_lds_dwordx4 %1, off nt\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(g), "s"(lds)
        : "memory");
  } else {
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "global_load_lds_dwordx4 %1, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(g), "s"(lds)
        : "memory");
  }
}

// Wait until at most N vector-memory operations of this wave are in flight,
// then join the workgroup barrier (no implicit drain, no fence).
template <int N>
__device__ __forceinline__ void ring_wait_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" : : "n"(N) : "memory");
}

__device__ __forceinline__ void vm_drain() { asm volatile("s_waitcnt vmcnt(0)" : : : "memory"); }

// Shared-tile variant (bf16): the four waves of a workgroup own four row
// groups (128 requests) of one vocabulary chunk, walked in steps of NT
// 16-wide tiles.  Every byte of a step -- NT W2 tiles (one contiguous block
// in HBM) and each wave's U (and, for the residual, target) rows -- is moved
// by direct global->LDS loads (global_load_lds_dwordx4: no register
// staging), D steps ahead, into a ring of D + 1 LDS slots.  Before a step
// each wave waits until its own loads of that step have landed (vmcnt counts
// the later steps still in flight), then a barrier makes every wave's share
// visible.  With NT = 2 a row load moves 128 contiguous bytes of each of 8
// rows: loads that touch 16 rows of 64 bytes each stream markedly slower.
//
// LDS layouts are XOR-swizzled instead of padded (a load writes 1 KB
// contiguously per wave): 16-byte chunk c of W2 tile row r is stored at
// chunk c ^ (r & 15); float4 c of U row j at c ^ ((j >> (2 / NT)) & (4 NT - 1)).
// Both make the 16 lanes of a ds_read_b128 phase hit disjoint banks.
template <int R, int MODE, int D, int NT, int HS>
__global__ __launch_bounds__(256) void sweep_shared_impl(const SweepArgs a) {
  using WR = WaveRows<uint16_t, R, MODE, HS>;
  using FragT = typename WR::FragT;
  constexpr int NS = WR::NS;
  constexpr int NB = D + 1;                             // ring slots
  constexpr int kRowBytes = R * 2;
  constexpr int kCPR = kRowBytes / 16;                  // 16-byte chunks per W2 row
  constexpr int kTileBytes = kTileV * kRowBytes;
  constexpr int kW2Bytes = NT * kTileBytes;             // W2 per step
  constexpr int kW2Inst = kW2Bytes / (kWavesPerBlock * 1024);   // 1 KB per wave instruction
  constexpr bool kResid = MODE == kModeResidual || MODE == kModeAlpha;   // target rows ride along
  constexpr int kFPR = 4 * NT;                          // float4 per U row per step
  constexpr int kRPI = 16 / NT;                         // U rows per load instruction
  constexpr int kSwzShift = 2 / NT;
  constexpr int kUInst = kRowsPerWave / kRPI;           // per wave per step (= 2 NT)
  constexpr int kWaveRowBytes = kRowsPerWave * kFPR * 16;
  constexpr int kG = kW2Inst + kUInst * (kResid ? 2 : 1);   // loads per wave per step
  constexpr int kUOff = kW2Bytes;
  constexpr int kTOff = kW2Bytes + kWavesPerBlock * kWaveRowBytes;
  constexpr int kSlotBytes = kW2Bytes + kWavesPerBlock * kWaveRowBytes * (kResid ? 2 : 1);
  static_assert(NT == 1 || NT == 2, "steps of one or two tiles");
  static_assert(kW2Inst >= 1 && kW2Bytes % (kWavesPerBlock * 1024) == 0, "W2 step must split into 1 KB loads");
  static_assert(D >= 1 && (D - 1) * kG < 64, "ring depth");
  __shared__ __attribute__((aligned(16))) unsigned char ring[NB * kSlotBytes];

  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int q = lane >> 4;
  const int j = lane & 15;
  const int blk = a.xcd_remap ? xcd_logical_block(blockIdx.x, gridDim.x) : (int)blockIdx.x;
  const int n_rq = (a.n_rg + kWavesPerBlock - 1) / kWavesPerBlock;
  const int g = blk % n_rq;
  const int vc = blk / n_rq;
  if (vc >= a.n_vc) return;                              // uniform over the block
  WR w;
  w.setup_rows(a, g * kWavesPerBlock + wid, j);
  const bool wave_active = __any(w.ok[0] || w.ok[1]);
  if constexpr (MODE == kModeResidual) {
    if (!__syncthreads_or(wave_active)) return;          // uniform over the block
  }
  LaneState st[2];
  lane_init(st[0]);
  lane_init(st[1]);
  // chunk boundaries on whole steps; only the last chunk may end mid-step
  const int n_steps = (a.n_tiles + NT - 1) / NT;
  const int t0 = min(NT * (int)((int64_t)n_steps * vc / a.n_vc), a.n_tiles);
  const int t1 = min(NT * (int)((int64_t)n_steps * (vc + 1) / a.n_vc), a.n_tiles);
  if (t0 >= t1) {
    w.setup_rest(a, q);
    w.finish(a, st, q, vc);
    return;
  }

  // Load lane roles.  W2: lane of instruction p fills LDS chunk
  // P = (wid kW2Inst + p) 64 + lane of the step.  Rows: lane i of row load m
  // fills row m kRPI + i / kFPR, float4 slot i % kFPR, which holds logical
  // float4 (i % kFPR) ^ swizzle(row); row offsets come from the MFMA lane
  // holding that row.
  int64_t uoff_d[kUInst], toff_d[kUInst];
  int ucol_d[kUInst];
#pragma unroll
  for (int m = 0; m < kUInst; ++m) {
    const int row = m * kRPI + lane / kFPR;
    ucol_d[m] = 4 * ((lane % kFPR) ^ ((row >> kSwzShift) & (kFPR - 1)));
    uoff_d[m] = __shfl(w.uoff[row >> 4], row & 15, 64);
    toff_d[m] = kResid ? __shfl(w.toff[row >> 4], row & 15, 64) : 0;
  }
  const unsigned char* W2b = static_cast<const unsigned char*>(a.W2);
  const uint32_t ring_lds = (uint32_t)(uintptr_t)(lds_u8_t*)ring;
  const uint32_t w2_lds = __builtin_amdgcn_readfirstlane(wid * kW2Inst * 1024);
  const uint32_t u_lds = __builtin_amdgcn_readfirstlane(kUOff + wid * kWaveRowBytes);
  const uint32_t t_lds = __builtin_amdgcn_readfirstlane(kTOff + wid * kWaveRowBytes);
  // step at tile t (t0 + a multiple of NT): tiles t .. t+NT-1; addresses
  // past the chunk are clamped into it (in bounds; those values are unused)
  auto issue = [&](int t, int sidx) {
    const uint32_t base = ring_lds + sidx * kSlotBytes;
#pragma unroll
    for (int p = 0; p < kW2Inst; ++p) {
      const int P = (wid * kW2Inst + p) * 64 + lane;
      const int r = P / kCPR;                            // row of the step, 0 .. 16 NT - 1
      const int c = (P % kCPR) ^ (r & 15);
      const int tc = min(t + r / kTileV, t1 - 1);
      dma16(W2b + (int64_t)tc * kTileBytes + (r % kTileV) * kRowBytes + c * 16, base + w2_lds + p * 1024);
    }
    int vcol[kUInst];
#pragma unroll
    for (int m = 0; m < kUInst; ++m) vcol[m] = min(t * kTileV + ucol_d[m], t1 * kTileV - 4);
#pragma unroll
    for (int m = 0; m < kUInst; ++m) dma16(a.U + uoff_d[m] + vcol[m], base + u_lds + m * 1024);
    if constexpr (kResid) {
#pragma unroll
      for (int m = 0; m < kUInst; ++m) dma16(a.T + toff_d[m] + vcol[m], base + t_lds + m * 1024);
    }
  };
  // operands of tile h of the step in slot sl
  auto load_tile = [&](int h, const unsigned char* sl, FragT (&A)[NS], float4 (&uu)[2], float4 (&tt)[2]) {
    const unsigned char* row = sl + (h * kTileV + j) * kRowBytes;
#pragma unroll
    for (int s = 0; s < NS; ++s) A[s] = *reinterpret_cast<const FragT*>(row + (((4 * s + q) ^ j) * 16));
    const int col = (4 * h + q) ^ ((j >> kSwzShift) & (kFPR - 1));
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int off = wid * kWaveRowBytes + ((nb * 16 + j) * kFPR + col) * 16;
      uu[nb] = *reinterpret_cast<const float4*>(sl + kUOff + off);
      if constexpr (kResid)
        tt[nb] = *reinterpret_cast<const float4*>(sl + kTOff + off);
      else
        tt[nb] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  auto compute = [&](int t, const unsigned char* sl) {
    if constexpr (!kResid && NT == 2 && HS == 0) {
      // Markov draft: both tiles through the MFMA, then one fold for the
      // step (the GRU head, whose state fragments are twice as many, folds
      // tile by tile below: its two-tile fold would need a second wave's
      // registers)
      f32x4_t acc[NT][2];
      FragT A[NS];
      float4 uu[2], tt[2];
      load_tile(0, sl, A, uu, tt);
      w.mma_tile(acc[0], A, uu);
      if (t + 1 < t1) {                                  // uniform over the block
        load_tile(1, sl, A, uu, tt);
        w.mma_tile(acc[1], A, uu);
        w.template fold<2>(a, st, acc, t, q);
      } else {
        const f32x4_t acc1[1][2] = {{acc[0][0], acc[0][1]}};
        w.template fold<1>(a, st, acc1, t, q);
      }
    } else {
#pragma unroll
      for (int h = 0; h < NT; ++h) {
        if (t + h >= t1) break;                          // uniform over the block
        FragT A[NS];
        float4 uu[2], tt[2];
        load_tile(h, sl, A, uu, tt);
        w.compute(a, st, t + h, q, A, uu, tt);
      }
    }
  };

  // First loads go out before the W1 gathers so both latencies overlap.
#pragma unroll
  for (int p = 0; p < D; ++p) issue(t0 + p * NT, p);
  w.setup_rest(a, q);
  // Drain once, visibly to the compiler: the set-up loads (W1 rows, tokens)
  // are then complete, and it places no waits for them inside the loop --
  // such a wait would also drain the ring there.
  __builtin_amdgcn_s_waitcnt(0xF70);
  for (int t = t0; t < t1; t += NB * NT) {
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int ts = t + u * NT;
      if (ts >= t1) break;                               // uniform over the block
      // this wave's loads of step ts have landed (the D-1 later steps may
      // still be in flight); after the barrier so have every other wave's,
      // and no wave still reads the slot that the next load overwrites
      ring_wait_barrier<(D - 1) * kG>();
      issue(ts + D * NT, (u + D) % NB);
      if (wave_active) compute(ts, ring + u * kSlotBytes);
    }
  }
  vm_drain();                                            // no load in flight at exit
  w.finish(a, st, q, vc);
}

// Chained draft (Markov head, bf16, one request quad: B <= 128): every
// position in one launch.  The work items (position k, vocabulary chunk) are
// those of the per-position shared-tile sweep, claimed from one ticket
// counter in (k, chunk) order by a grid of persistent workgroups.  An item
// of position k first issues its first D ring steps (U and W2 do not depend
// on the tokens), then waits until every item of position k - 1 has
// published its chunk winners, then takes x_{k-1} from the slot groups,
// gathers the W1 rows and runs the sweep.  Items are claimed in dependency
// order and a workgroup finishes its item before it claims the next, so
// every item waited on is held by a running workgroup: the launch never
// depends on how many of its workgroups are resident (concurrent kernels
// only slow it down).  The wait is bounded all the same (it raises the
// barrier error bit and lets the item run on).
//
// The requests form one or two groups of 64 or 128 rows (NBW = 1 or 2
// 16-row blocks per wave); each group is its own chain of positions, and
// tickets interleave the groups (position-major), so while one group waits
// for its previous position the other group's items keep the device
// streaming.
//
// Counters (zero at launch; the draft combine clears them): chain[0] the
// ticket counter, chain[32 + kg] the finished items of (position, group) kg
// (another cache line).  The workgroup whose item completes (k, g) releases
// the waiting workgroups by writing k into word g of each one's own flag line
// (flags[32 b + g], one 128-byte line per workgroup): hundreds of workgroups
// polling one counter slowed the streaming of the ones still working
// (straggling items took twice the median time).  The item that completes a
// group's last position writes 0 into that group's flags, so each launch (a
// graph replay too) starts from zeroed flags.
constexpr unsigned kChainSpinLimit = 1u << 20;

template <int R, int MODE, int D, int NT, int NBW, int NW>
__global__ __launch_bounds__(64 * NW) void draft_chain_impl(const SweepArgs a0) {
  using WR = WaveRows<uint16_t, R, MODE, 0, NBW>;
  using FragT = typename WR::FragT;
  constexpr int NS = WR::NS;
  constexpr int NB = D + 1;
  constexpr int kRowsW = WR::kRows;                     // request rows per wave
  constexpr int kRowsItem = NW * kRowsW;    // request rows per item (one group)
  constexpr int kRowBytes = R * 2;
  constexpr int kCPR = kRowBytes / 16;
  constexpr int kTileBytes = kTileV * kRowBytes;
  constexpr int kW2Bytes = NT * kTileBytes;
  constexpr int kW2Inst = kW2Bytes / (NW * 1024);
  constexpr int kFPR = 4 * NT;
  constexpr int kRPI = 16 / NT;
  constexpr int kSwzShift = 2 / NT;
  constexpr int kUInst = kRowsW / kRPI;
  constexpr int kWaveRowBytes = kRowsW * kFPR * 16;
  constexpr int kG = kW2Inst + kUInst;
  constexpr int kUOff = kW2Bytes;
  constexpr int kSlotBytes = kW2Bytes + NW * kWaveRowBytes;
  static_assert(NT == 1 || NT == 2, "steps of one or two tiles");
  static_assert(NBW == 1 || NBW == 2, "one or two 16-row blocks per wave");
  static_assert(NW == 4 || NW == 8, "four or eight waves");
  static_assert(kW2Bytes % (NW * 1024) == 0, "W2 step must split into 1 KB loads per wave");
  static_assert(MODE == kModeDraftGreedy || MODE == kModeDraftSample, "draft modes only");
  static_assert(D >= 1 && (D - 1) * kG < 64, "ring depth");
  __shared__ __attribute__((aligned(16))) unsigned char ring[NB * kSlotBytes];
  // the claimed ticket is handed to every wave through the last word of the
  // ring (one more LDS word could cost a resident workgroup per CU): that
  // word is first overwritten by the loop's first load into the last slot,
  // which follows a barrier every wave reaches after reading it
  int* const s_item = reinterpret_cast<int*>(ring + NB * kSlotBytes - 4);

  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int q = lane >> 4;
  const int j = lane & 15;
  const int n_grp = (a0.B + kRowsItem - 1) / kRowsItem;   // request groups, independent chains
  const int per_kg = a0.n_vc;                               // items of one (position, group)
  const int total = per_kg * n_grp * a0.gamma;
  const int n_steps = (a0.n_tiles + NT - 1) / NT;
  const unsigned char* W2b = static_cast<const unsigned char*>(a0.W2);
  const uint32_t ring_lds = (uint32_t)(uintptr_t)(lds_u8_t*)ring;
  const uint32_t w2_lds = __builtin_amdgcn_readfirstlane(wid * kW2Inst * 1024);
  const uint32_t u_lds = __builtin_amdgcn_readfirstlane(kUOff + wid * kWaveRowBytes);

  if (threadIdx.x == 0)
    *s_item = (int)__hip_atomic_fetch_add(a0.chain, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  int item = *s_item;
  while (item < total) {                                  // uniform over the block
    const int kg = item / per_kg;                         // (position, group), position-major
    const int k = kg / n_grp + 1;
    const int g = kg - (k - 1) * n_grp;
    const int vc = item - kg * per_kg;
    SweepArgs a = a0;
    a.k = k;
    a.pf = a0.pf + (size_t)(k - 1) * a0.B * a0.n_vc;
    a.pi = a0.pi + (size_t)(k - 1) * a0.B * a0.n_vc;
    a.best = a0.best + (size_t)(k - 1) * kBestGroups * a0.B;
    a.best_prev = k > 1 ? a0.best + (size_t)(k - 2) * kBestGroups * a0.B : nullptr;
    WR w;
    w.setup_rows(a, g * NW + wid, j);
    bool any_ok = false;
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) any_ok = any_ok || w.ok[nb];
    const bool wave_active = __any(any_ok);
    LaneState st[NBW];
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) lane_init(st[nb]);
    const int t0 = min(NT * (int)((int64_t)n_steps * vc / a.n_vc), a.n_tiles);
    const int t1 = min(NT * (int)((int64_t)n_steps * (vc + 1) / a.n_vc), a.n_tiles);

    int64_t uoff_d[kUInst];
    int ucol_d[kUInst];
#pragma unroll
    for (int m = 0; m < kUInst; ++m) {
      const int row = m * kRPI + lane / kFPR;
      ucol_d[m] = 4 * ((lane % kFPR) ^ ((row >> kSwzShift) & (kFPR - 1)));
      uoff_d[m] = __shfl(w.uoff[row >> 4], row & 15, 64);
    }
    auto issue = [&](int t, int sidx) {
      const uint32_t base = ring_lds + sidx * kSlotBytes;
#pragma unroll
      for (int p = 0; p < kW2Inst; ++p) {
        const int P = (wid * kW2Inst + p) * 64 + lane;
        const int r = P / kCPR;
        const int c = (P % kCPR) ^ (r & 15);
        const int tc = min(t + r / kTileV, t1 - 1);
        dma16(W2b + (int64_t)tc * kTileBytes + (r % kTileV) * kRowBytes + c * 16, base + w2_lds + p * 1024);
      }
      int vcol[kUInst];
#pragma unroll
      for (int m = 0; m < kUInst; ++m) vcol[m] = min(t * kTileV + ucol_d[m], t1 * kTileV - 4);
#pragma unroll
      for (int m = 0; m < kUInst; ++m) dma16<true>(a.U + uoff_d[m] + vcol[m], base + u_lds + m * 1024);
    };
    auto load_tile = [&](int h, const unsigned char* sl, FragT (&A)[NS], float4 (&uu)[NBW]) {
      const unsigned char* row = sl + (h * kTileV + j) * kRowBytes;
#pragma unroll
      for (int s2 = 0; s2 < NS; ++s2) A[s2] = *reinterpret_cast<const FragT*>(row + (((4 * s2 + q) ^ j) * 16));
      const int col = (4 * h + q) ^ ((j >> kSwzShift) & (kFPR - 1));
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) {
        const int off = wid * kWaveRowBytes + ((nb * 16 + j) * kFPR + col) * 16;
        uu[nb] = *reinterpret_cast<const float4*>(sl + kUOff + off);
      }
    };
    auto compute = [&](int t, const unsigned char* sl) {
      if constexpr (NT == 2) {
        f32x4_t acc[NT][NBW];
        FragT A[NS];
        float4 uu[NBW];
        load_tile(0, sl, A, uu);
        w.mma_tile(acc[0], A, uu);
        if (t + 1 < t1) {                                  // uniform over the block
          load_tile(1, sl, A, uu);
          w.mma_tile(acc[1], A, uu);
          w.template fold<2>(a, st, acc, t, q);
        } else {
          f32x4_t acc1[1][NBW];
#pragma unroll
          for (int nb = 0; nb < NBW; ++nb) acc1[0][nb] = acc[0][nb];
          w.template fold<1>(a, st, acc1, t, q);
        }
      } else {
        f32x4_t acc[1][NBW];
        FragT A[NS];
        float4 uu[NBW];
        load_tile(0, sl, A, uu);
        w.mma_tile(acc[0], A, uu);
        w.template fold<1>(a, st, acc, t, q);
      }
    };

    if (t0 < t1) {
#pragma unroll
      for (int p = 0; p < D; ++p) issue(t0 + p * NT, p);
    }
    // every item of (k - 1, g) has published its winners
    if (k > 1) {
      if (threadIdx.x == 0) {
        // the host's failure injection waits for a value nobody writes
        const unsigned want = a0.bar_test ? 0x80u : (unsigned)(k - 1);
        const unsigned limit = a0.bar_test ? 64u : kChainSpinLimit;
        const unsigned* flag = a0.chain_flags + 32 * blockIdx.x + g;
        unsigned spins = 0;
        while (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < want) {
          __builtin_amdgcn_s_sleep(2);
          if (++spins > limit) {
            atomicOr(a0.err, kErrBarrier);
            break;
          }
        }
      }
      __syncthreads();
    }
    w.template setup_rest<true>(a, q);
    // drain visibly to the compiler: the set-up loads and the first ring
    // steps are complete, and no wait for them lands inside the loop
    __builtin_amdgcn_s_waitcnt(0xF70);
    for (int t = t0; t < t1; t += NB * NT) {
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        const int ts = t + u * NT;
        if (ts >= t1) break;                               // uniform over the block
        ring_wait_barrier<(D - 1) * kG>();
        issue(ts + D * NT, (u + D) % NB);
        if (wave_active) compute(ts, ring + u * kSlotBytes);
      }
    }
    vm_drain();
    w.finish(a, st, q, vc);
    vm_drain();                                            // this wave's partials and slot atomics are done
    __syncthreads();                                       // every wave's; no wave reads the ring any more
    if (wid == 0) {
      unsigned before = 0;
      if (lane == 0)
        before = __hip_atomic_fetch_add(a0.chain + 32 + kg, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      before = __shfl(before, 0, 64);
      if (before == (unsigned)per_kg - 1u) {
        // the last item of (k, g): release every workgroup's wait on group g
        // (after the last position: clear the group's flags for the next launch)
        const unsigned v = k < a0.gamma ? (unsigned)k : 0u;
        for (int b = lane; b < (int)gridDim.x; b += 64)
          __hip_atomic_store(a0.chain_flags + 32 * b + g, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      if (lane == 0)
        *s_item = (int)__hip_atomic_fetch_add(a0.chain, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    item = *s_item;
  }
}

// Whole-draft variant (Markov head, bf16 weights, r = 256, B <= 128): one
// launch runs every position.  Each wave owns up to kPersistTiles 16-wide
// vocabulary tiles and keeps their W2 fragments (the MFMA A operand) in
// registers for the whole draft, so W2 is read from memory once per call
// instead of once per position; per position only U (and the W1 rows of the
// previous tokens) move.  One 4-wave workgroup per CU: its LDS (128 KB) and
// registers admit no second one per CU, so the grid of one per CU is resident
// at once on an otherwise idle device (the host can also launch it
// cooperatively); positions are separated by a grid barrier (an arrival
// counter with a bounded spin, so a workgroup that is not yet resident delays
// the barrier and never deadlocks it for good).
//
// Per position: the four waves gather the 128 W1 rows of the previous tokens
// into LDS (chunk c of row b at chunk c ^ (b & 15), which makes the B-operand
// reads conflict free); then each wave walks its steps (request block nb of
// 16 rows) x (tile pair p): U of the step (16 rows x 128 bytes) comes through
// a private ring of kPersistRing LDS slots filled by direct global->LDS loads
// that run up to kPersistRing - 1 steps ahead, across position boundaries
// (U does not depend on the tokens).  At the end of a request block the wave
// writes its partial and its slot-group atomic, exactly as a chunk of the
// per-position sweep does; the partials of every position are merged by the
// draft combine.
constexpr int kPersistRing = 8;
constexpr int kPersistSteps = 16 * 128;              // bytes of U per step
constexpr unsigned kSpinLimit = 1u << 20;            // polls before a barrier gives up

// Ring wait of the whole-draft kernel: a step's two loads have landed when at
// most the loads of the D - 1 = 6 later steps are in flight.
__device__ __forceinline__ void vm_wait12() { asm volatile("s_waitcnt vmcnt(12)" : : : "memory"); }

// Grid barrier: every workgroup adds one arrival after all its waves' slot
// atomics have completed; the counter starts at zero (the draft combine
// resets it).  The values that cross the barrier are the slot-group atomics,
// which are performed device-coherently, and they are read back with
// agent-scope atomic loads (coherent, no cached copy), so each wave only
// waits for its own memory operations (vmcnt 0) instead of a release fence:
// a release fence at agent scope writes back the L2 from every wave, which
// cost ~15 us per barrier here.  The partials written between barriers are
// read only by the next kernel.  A poll that never sees `target` gives up
// after kSpinLimit tries and raises the barrier error bit, so every wave
// always exits.
__device__ __forceinline__ void grid_barrier(unsigned int* bar, unsigned int target, unsigned int limit,
                                             int32_t* err) {
  vm_drain();
  __syncthreads();
  if (threadIdx.x == 0) {
    __hip_atomic_fetch_add(bar, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    unsigned spins = 0;
    while (__hip_atomic_load(bar, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
      __builtin_amdgcn_s_sleep(2);
      if (++spins > limit) {
        atomicOr(err, kErrBarrier);
        break;
      }
    }
  }
  __syncthreads();
}

template <int MODE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void draft_persist_impl(const SweepArgs a) {
  constexpr int R = 256;
  using F = Frag<uint16_t, R>;
  using FragT = typename F::T;
  constexpr int NS = F::NS;
  constexpr int TW = kPersistTiles;
  constexpr int NP = (TW + 1) / 2;
  constexpr int NBUF = kPersistRing;
  constexpr int D = NBUF - 1;
  static_assert(NBUF == 8 && 2 * (D - 1) == 12, "vm_wait12 assumes 8 slots of two loads");
  static_assert(TW % 2 == 0, "tiles come in pairs");
  __shared__ __attribute__((aligned(16))) unsigned char hbuf[128 * R * 2];
  __shared__ __attribute__((aligned(16))) unsigned char uring[kWavesPerBlock * NBUF * kPersistSteps];

  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: LDS bases go to M0
  const int q = lane >> 4;
  const int j = lane & 15;
  const int nw = gridDim.x * kWavesPerBlock;           // = n_vc: one chunk per wave
  const int wg = blockIdx.x * kWavesPerBlock + wid;
  const int t0 = (int)((int64_t)a.n_tiles * wg / nw);
  const int t1 = (int)((int64_t)a.n_tiles * (wg + 1) / nw);
  const int ntw = t1 - t0;                             // 0 .. TW (checked by the host)
  const int np = (ntw + 1) / 2;                        // tile pairs = steps per request block
  const int nbq = (a.B + 15) / 16;                     // request blocks
  const uint16_t* W2 = static_cast<const uint16_t*>(a.W2);
  const uint16_t* W1 = static_cast<const uint16_t*>(a.W1);

  // W2 fragments of the wave's tiles (tiles past the range repeat the last
  // tile of the vocabulary; they are never used)
  FragT A[TW][NS];
#pragma unroll
  for (int t = 0; t < TW; ++t) {
    const int tt = min(t0 + t, a.n_tiles - 1);
    const uint16_t* row = W2 + ((int64_t)tt * kTileV + j) * R;
#pragma unroll
    for (int s = 0; s < NS; ++s) A[t][s] = F::load(row, s, q);
  }
  // request ids of rows lane and lane + 64 (stream keys, sampling)
  uint32_t rid[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int b = lane + 64 * h;
    rid[h] = (b < a.B) ? (a.req ? a.req[b] : (uint32_t)b) : 0u;
  }

  // ring cursor: the next step to load, as (position, request block, pair)
  const uint32_t ring_lds =
      __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_u8_t*)uring + wid * NBUF * kPersistSteps);
  int ik = 1, inb = 0, ip = 0, gi = 0;
  const bool has_steps = np > 0;
  auto issue_next = [&]() {
    if (!has_steps || ik > a.gamma) return;            // uniform over the wave
    const uint32_t dst = ring_lds + (gi & (NBUF - 1)) * kPersistSteps;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int r = m * 8 + (lane >> 3);
      const int b = inb * 16 + r;
      const int c = (lane & 7) ^ ((r >> 1) & 7);
      const int col = min((t0 + 2 * ip) * kTileV + 4 * c, t1 * kTileV - 4);
      const float* src = a.U + (b < a.B ? (int64_t)b * a.usb : 0) + (int64_t)(ik - 1) * a.usk + col;
      dma16(src, dst + m * 1024);
    }
    ++gi;
    if (++ip == np) {
      ip = 0;
      if (++inb == nbq) {
        inb = 0;
        ++ik;
      }
    }
  };
#pragma unroll
  for (int d = 0; d < D; ++d) issue_next();

  const uint32_t h_lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_u8_t*)hbuf);
  int gs = 0;                                          // next step to consume
  for (int k = 1; k <= a.gamma; ++k) {
    // previous tokens of rows wid*32 + (lane & 31): the anchor, or the
    // maximum over the previous position's slot groups (each half-wave reads
    // eight groups)
    {
      const int rq = wid * 32 + (lane & 31);
      const bool act = rq < a.B;
      int tok = 0;
      if (k == 1) {
        tok = act ? a.anchor[rq] : 0;
      } else {
        unsigned long long pb = 0ull;
        if (act) {
          const unsigned long long* bp = a.best + (int64_t)(k - 2) * kBestGroups * a.B;
#pragma unroll
          for (int i = 0; i < kBestGroups / 2; ++i) {
            const unsigned long long v = __hip_atomic_load(
                bp + (int64_t)((lane >> 5) * (kBestGroups / 2) + i) * a.B + rq, __ATOMIC_RELAXED,
                __HIP_MEMORY_SCOPE_AGENT);
            pb = v > pb ? v : pb;
          }
        }
        const unsigned long long o = __shfl_xor(pb, 32, 64);
        pb = o > pb ? o : pb;
        tok = act ? best_index(pb) : 0;
      }
      if ((unsigned)tok >= (unsigned)a.V) {
        atomicOr(a.err, kErrToken);
        tok = 0;
      }
      // gather: instruction i fills rows 2i and 2i + 1 of the wave's quarter
      // (1 KB of LDS); lane L writes chunk slot L & 31 of its row, which
      // holds chunk (L & 31) ^ (row & 15)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int rr = 2 * i + (lane >> 5);
        const int b = wid * 32 + rr;
        const int tk = __shfl(tok, rr, 64);
        const int c = (lane & 31) ^ (b & 15);
        dma16(W1 + (int64_t)tk * R + c * 8, h_lds + (wid * 32 + 2 * i) * 512);
      }
      vm_drain();
      __syncthreads();
    }

    for (int nb = 0; nb < nbq; ++nb) {
      const int b = nb * 16 + j;
      const bool ok = b < a.B;
      uint32_t klo = 0u, khi = 0u;
      if constexpr (MODE == kModeDraftSample) {
        const uint32_t r0 = __shfl(rid[0], b & 63, 64), r1 = __shfl(rid[1], b & 63, 64);
        const uint64_t key = stream_key(a.seed, b < 64 ? r0 : r1, (uint32_t)k, kDraft);
        klo = (uint32_t)key;
        khi = (uint32_t)(key >> 32);
      }
      FragT Hf[NS];
#pragma unroll
      for (int s = 0; s < NS; ++s)
        Hf[s] = *reinterpret_cast<const FragT*>(hbuf + (nb * 16 + j) * 512 + (((4 * s + q) ^ j) * 16));
      LaneState st;
      lane_init(st);
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        if (p >= np) break;                              // uniform over the wave
        // this step's loads have landed when at most the D - 1 later steps
        // (two loads each) are in flight
        vm_wait12();
        issue_next();
        const unsigned char* sl = uring + wid * NBUF * kPersistSteps + (gs & (NBUF - 1)) * kPersistSteps;
        ++gs;
        f32x4_t acc[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int c = (4 * h + q) ^ ((j >> 1) & 7);
          const float4 u = *reinterpret_cast<const float4*>(sl + j * 128 + c * 16);
          acc[h] = f32x4_t{u.x, u.y, u.z, u.w};
        }
#pragma unroll
        for (int s = 0; s < NS; ++s) acc[0] = F::mma(A[2 * p][s], Hf[s], acc[0]);
        const int v0 = (t0 + 2 * p) * kTileV + 4 * q;
        if (2 * p + 1 < ntw) {                           // uniform over the wave
#pragma unroll
          for (int s = 0; s < NS; ++s) acc[1] = F::mma(A[2 * p + 1][s], Hf[s], acc[1]);
          const f32x4_t z2[2] = {acc[0], acc[1]};
          fold_draft<MODE, 2>(st, z2, v0, klo, khi, a.s2);
        } else {
          const f32x4_t z1[1] = {acc[0]};
          fold_draft<MODE, 1>(st, z1, v0, klo, khi, a.s2);
        }
      }
      resolve_draft<MODE>(st, klo, khi, a.s2);
      lane_merge<MODE>(st, 16);
      lane_merge<MODE>(st, 32);
      if (q == 0 && ok) {
        const int64_t o = ((int64_t)(k - 1) * a.B + b) * nw + wg;
        a.pf[o] = make_float4(st.m, st.s, st.key, st.zb);
        a.pi[o] = make_int2(st.idx, 0);
        unsigned long long* slot = a.best + ((int64_t)(k - 1) * kBestGroups + (wg % kBestGroups)) * a.B + b;
        __hip_atomic_fetch_max(slot, pack_best(st.key, st.idx), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    if (k < a.gamma)
      grid_barrier(a.bar, (unsigned)gridDim.x * (unsigned)k + (a.bar_test ? 1u : 0u), a.bar_test ? 64u : kSpinLimit,
                   a.err);
  }
  vm_drain();                                            // no load in flight at exit
}

constexpr int kCombineThreads = 256;

// One 256-thread workgroup per (request, position), after the whole draft
// loop: merge the per-chunk partials in a fixed order, write x_k, the
// log-normaliser and y at x_k, and clear the position's running best (the
// sweeps already took x_k from it; it must be zero for the next call).
__global__ __launch_bounds__(kCombineThreads) void combine_draft_impl(const CombineArgs a) {
  const int b = blockIdx.x;
  const int k = blockIdx.y + 1;
  DraftPart p{-INFINITY, 0.f, -INFINITY, 0.f, 0x7fffffff};
  const int64_t base = ((int64_t)(k - 1) * a.B + b) * a.n_vc;
  for (int i = threadIdx.x; i < a.n_vc; i += kCombineThreads) {
    const float4 f = a.pf[base + i];
    part_merge(p, DraftPart{f.x, f.y, f.z, f.w, a.pi[base + i].x});
  }
#pragma unroll
  for (int mask = 1; mask < 64; mask <<= 1) part_merge(p, part_shfl(p, mask));
  __shared__ DraftPart red[kCombineThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = p;
  __syncthreads();
  if (threadIdx.x == 0) {
#pragma unroll
    for (int w = 1; w < kCombineThreads / 64; ++w) part_merge(p, red[w]);
    int idx = p.idx;
    if ((unsigned)idx >= (unsigned)a.V) {
      atomicOr(a.err, kErrToken);
      idx = 0;
    }
    const int64_t o = (int64_t)b * a.gamma + k - 1;
    a.tokens[o] = idx;
    a.lse[o] = (p.m + fast_log2(p.s)) * kLn2;
    a.ytok[o] = a.greedy ? p.key : p.zb;   // sampling partials carry y itself
  }
  if (a.bar && b == 0 && k == 1 && threadIdx.x == 0) *a.bar = 0u;   // grid barrier of the whole-draft kernel
  if (a.chain && b == 0 && k == 1 && threadIdx.x < 97)   // chained draft counters
    a.chain[threadIdx.x == 0 ? 0 : 31 + threadIdx.x] = 0u;
  if (a.best && threadIdx.x < kBestGroups) {
    unsigned long long* slot = a.best + ((int64_t)(k - 1) * kBestGroups + threadIdx.x) * a.B + b;
    __hip_atomic_store(slot, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

struct ResidPart {
  float key, fkey;
  int idx, fidx;
};

__device__ __forceinline__ void resid_merge(ResidPart& a, const ResidPart& b) {
  if (key_beats(b.key, b.idx, a.key, a.idx)) {
    a.key = b.key;
    a.idx = b.idx;
  }
  if (key_beats(b.fkey, b.fidx, a.fkey, a.fidx)) {
    a.fkey = b.fkey;
    a.fidx = b.fidx;
  }
}

// One workgroup per request with a pending residual draw: merge its partials
// and write the emitted token after the accepted prefix.
__global__ __launch_bounds__(kCombineThreads) void combine_resid_impl(const CombineArgs a) {
  const int b = blockIdx.x;
  if (a.resid_k[b] <= 0) return;
  ResidPart p{-INFINITY, -INFINITY, 0x7fffffff, 0x7fffffff};
  const int64_t base = (int64_t)b * a.n_vc;
  for (int i = threadIdx.x; i < a.n_vc; i += kCombineThreads) {
    const float4 f = a.pf[base + i];
    const int2 pi = a.pi[base + i];
    resid_merge(p, ResidPart{f.x, f.y, pi.x, pi.y});
  }
#pragma unroll
  for (int mask = 1; mask < 64; mask <<= 1)
    resid_merge(p, ResidPart{shfl_xor(p.key, mask), shfl_xor(p.fkey, mask), shfl_xor(p.idx, mask),
                             shfl_xor(p.fidx, mask)});
  __shared__ ResidPart red[kCombineThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = p;
  __syncthreads();
  if (threadIdx.x == 0) {
#pragma unroll
    for (int w = 1; w < kCombineThreads / 64; ++w) resid_merge(p, red[w]);
    int tok = (p.key > -INFINITY) ? p.idx : p.fidx;
    if ((unsigned)tok >= (unsigned)a.V) {
      atomicOr(a.err, kErrToken);
      tok = 0;
    }
    const int A = a.accept_len[b];
    if ((unsigned)A > (unsigned)a.gamma) {               // only after a failed verification
      atomicOr(a.err, kErrK);
      return;
    }
    a.out_tokens[(int64_t)b * (a.gamma + 1) + A] = tok;
  }
}

// One 256-thread workgroup per (request, position): the acceptance
// probability of the position is the sum of its chunk partials.
__global__ __launch_bounds__(kCombineThreads) void combine_alpha_impl(const CombineArgs a) {
  const int b = blockIdx.x;
  const int k = blockIdx.y + 1;
  const int64_t base = ((int64_t)(k - 1) * a.B + b) * a.n_vc;
  float acc = 0.0f;
  for (int i = threadIdx.x; i < a.n_vc; i += kCombineThreads) acc += a.pf[base + i].x;
#pragma unroll
  for (int mask = 1; mask < 64; mask <<= 1) acc += shfl_xor(acc, mask);
  __shared__ float red[kCombineThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    float tot = 0.0f;
#pragma unroll
    for (int w = 0; w < kCombineThreads / 64; ++w) tot += red[w];
    a.lse[(int64_t)b * a.gamma + k - 1] = tot;      // the alpha output
  }
}

template <int R, int D, int NT, int HS>
const void* shared_for(int mode) {
  if (mode == kModeDraftGreedy) return (const void*)&sweep_shared_impl<R, kModeDraftGreedy, D, NT, HS>;
  if (mode == kModeDraftSample) return (const void*)&sweep_shared_impl<R, kModeDraftSample, D, NT, HS>;
  if (mode == kModeResidual) return (const void*)&sweep_shared_impl<R, kModeResidual, D, NT, HS>;
  if (mode == kModeAlpha) return (const void*)&sweep_shared_impl<R, kModeAlpha, D, NT, HS>;
  return nullptr;
}

template <int D, int NT, int HS>
const void* shared_for_r(int r, int mode) {
  if (r == 128) return shared_for<128, D, NT, HS>(mode);
  if (r == 256) return shared_for<256, D, NT, HS>(mode);
  return nullptr;
}

template <int HS>
const void* shared_for_ring(int r, int mode, int depth, int nt) {
  if (nt == 1) {
    if (depth == 1) return shared_for_r<1, 1, HS>(r, mode);
    if (depth == 2) return shared_for_r<2, 1, HS>(r, mode);
    if (depth == 3) return shared_for_r<3, 1, HS>(r, mode);
  } else if (nt == 2) {
    if (depth == 1) return shared_for_r<1, 2, HS>(r, mode);
    if (depth == 2) return shared_for_r<2, 2, HS>(r, mode);
  }
  return nullptr;
}

template <typename WT, int R, int HS>
const void* private_for(int mode) {
  if (mode == kModeDraftGreedy) return (const void*)&sweep_private_impl<WT, R, kModeDraftGreedy, HS>;
  if (mode == kModeDraftSample) return (const void*)&sweep_private_impl<WT, R, kModeDraftSample, HS>;
  if (mode == kModeResidual) return (const void*)&sweep_private_impl<WT, R, kModeResidual, HS>;
  if (mode == kModeAlpha) return (const void*)&sweep_private_impl<WT, R, kModeAlpha, HS>;
  return nullptr;
}

template <typename WT, int HS>
const void* private_for_r(int r, int mode) {
  switch (r) {
    case 32: return private_for<WT, 32, HS>(mode);
    case 64: return private_for<WT, 64, HS>(mode);
    case 128: return private_for<WT, 128, HS>(mode);
    case 256: return private_for<WT, 256, HS>(mode);
    default: return nullptr;
  }
}

}  // namespace

const void* sweep_kernel(int wdtype, int r, int mode, int depth, int nt, int hs) {
  if (depth) {
    if (wdtype != 1) return nullptr;
    return hs ? shared_for_ring<1>(r, mode, depth, nt) : shared_for_ring<0>(r, mode, depth, nt);
  }
  if (wdtype == 1) return hs ? private_for_r<uint16_t, 1>(r, mode) : private_for_r<uint16_t, 0>(r, mode);
  if (wdtype == 0) return hs ? private_for_r<float, 1>(r, mode) : private_for_r<float, 0>(r, mode);
  return nullptr;
}

template <int R, int D, int NT, int NBW, int NW>
const void* chain_for(int mode) {
  return mode == kModeDraftGreedy ? (const void*)&draft_chain_impl<R, kModeDraftGreedy, D, NT, NBW, NW>
                                  : (const void*)&draft_chain_impl<R, kModeDraftSample, D, NT, NBW, NW>;
}

const void* draft_chain_kernel(int r, int mode, int depth, int nt, int rows_per_wave, int waves) {
  if (mode != kModeDraftGreedy && mode != kModeDraftSample) return nullptr;
  if (waves == 4 && rows_per_wave == 32) {
    if (r == 256 && nt == 2 && depth == 1) return chain_for<256, 1, 2, 2, 4>(mode);
    if (r == 256 && nt == 1 && depth == 2) return chain_for<256, 2, 1, 2, 4>(mode);
    if (r == 128 && nt == 2 && depth == 1) return chain_for<128, 1, 2, 2, 4>(mode);
  } else if (waves == 4 && rows_per_wave == 16) {
    if (r == 256 && nt == 2 && depth == 1) return chain_for<256, 1, 2, 1, 4>(mode);
    if (r == 128 && nt == 2 && depth == 1) return chain_for<128, 1, 2, 1, 4>(mode);
  } else if (waves == 8 && rows_per_wave == 16) {
    if (r == 256 && nt == 2 && depth == 2) return chain_for<256, 2, 2, 1, 8>(mode);
    if (r == 256 && nt == 2 && depth == 3) return chain_for<256, 3, 2, 1, 8>(mode);
    if (r == 256 && nt == 2 && depth == 4) return chain_for<256, 4, 2, 1, 8>(mode);
    if (r == 128 && nt == 2 && depth == 2) return chain_for<128, 2, 2, 1, 8>(mode);
  }
  return nullptr;
}

const void* draft_persist_kernel(int mode) {
  if (mode == kModeDraftGreedy) return (const void*)&draft_persist_impl<kModeDraftGreedy>;
  if (mode == kModeDraftSample) return (const void*)&draft_persist_impl<kModeDraftSample>;
  return nullptr;
}

const void* combine_draft_kernel() { return (const void*)&combine_draft_impl; }
const void* combine_resid_kernel() { return (const void*)&combine_resid_impl; }
const void* combine_alpha_kernel() { return (const void*)&combine_alpha_impl; }

}  // namespace dspark
