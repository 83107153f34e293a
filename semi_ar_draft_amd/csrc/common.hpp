// Shared device helpers of libdspark: counter-based hash, bf16 fragments,
// base-2 online softmax and arg-max merge rules.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dspark {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

// Purposes of the random streams.
constexpr uint32_t kDraft = 1, kAccept = 2, kResid = 3, kBonus = 4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Device error flag bits.
constexpr int kErrToken = 1;    // a token id outside [0, V)
constexpr int kErrK = 2;        // a verify length outside [0, gamma]
constexpr int kErrRow = 4;      // a packed target row outside [0, n_rows)
constexpr int kErrBarrier = 8;  // a grid barrier of the whole-draft kernel gave up waiting
constexpr int kErrGrid = 16;    // a candidate temperature that is not positive and finite
constexpr int kErrLen = 32;     // an accepted length outside [0, gamma] (temperature fit)

// Element offset of target row (b, k) (k 1-based): strided [B][gamma+1][V]
// placement, or the packed layout where request b's rows 1 .. K_b + 1 start
// at row toffs[b] of an array of n_rows rows.  A packed row outside the
// array is flagged and replaced by row 0 (in bounds; results then invalid).
__device__ __forceinline__ int64_t target_row(const int32_t* toffs, int n_rows, int64_t tsb, int64_t tsk, int b,
                                              int k, int32_t* err) {
  if (!toffs) return (int64_t)b * tsb + (int64_t)(k - 1) * tsk;
  int64_t r = (int64_t)toffs[b] + (k - 1);
  if (r < 0 || r >= n_rows) {
    atomicOr(err, kErrRow);
    r = 0;
  }
  return r * tsk;
}

// ---------------------------------------------------------------------------
// Counter-based random numbers.
//
// Row key: the output function of SplitMix64 (Steele, Lea & Flood, 2014) is
// applied three times, folding in the request id, then (position << 8 |
// purpose).  Element v of a row: MurmurHash3's 32-bit finalizer of
// ((v * 0x9E3779B9) ^ lo(key)) + hi(key).  Uniform: (2 * (h >> 9) + 1) * 2^-24.
// ---------------------------------------------------------------------------
__host__ __device__ __forceinline__ uint64_t sm64_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__host__ __device__ __forceinline__ uint64_t stream_key(uint64_t seed, uint32_t req, uint32_t pos,
                                                        uint32_t purpose) {
  uint64_t k = sm64_mix(seed + 0x9E3779B97F4A7C15ull);
  k = sm64_mix(k ^ (uint64_t)req);
  return sm64_mix(k ^ (((uint64_t)pos << 8) | (uint64_t)purpose));
}

__device__ __forceinline__ uint32_t murmur_fmix32(uint32_t h) {
  h ^= h >> 16;
  h *= 0x85EBCA6Bu;
  h ^= h >> 13;
  h *= 0xC2B2AE35u;
  h ^= h >> 16;
  return h;
}

__device__ __forceinline__ uint32_t elem_hash(uint32_t klo, uint32_t khi, uint32_t v) {
  return murmur_fmix32(((v * 0x9E3779B9u) ^ klo) + khi);
}

// (2 * (h >> 9) + 1) * 2^-24, exact in fp32 (a single rounding of an exact value).
__device__ __forceinline__ float hash_uniform(uint32_t h) {
  return __builtin_fmaf((float)(h >> 9), 0x1.0p-23f, 0x1.0p-24f);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// ---------------------------------------------------------------------------
// Categorical draws by Gumbel-max.  Entry v of a row with weight w_v and
// uniform u_v has the key ln w_v - ln(-ln u_v); the draw is the lowest index
// attaining the largest key, so P(v) = w_v / sum w.  With E_v = -log2 u_v
// (a positive multiple of -ln u_v) the key order is the order of w_v / E_v,
// so a lane compares a candidate with its leader b as w_v E_b > w_b E_v
// (one logarithm per entry; the weights are the softmax terms already formed
// for the log-normaliser) and turns the leader into a log-domain key once,
// at the end of its range.
// ---------------------------------------------------------------------------
// E_v = -log2 u_v.  u_v = (2 (h >> 9) + 1) 2^-24 is formed as the float
// 1 + (h >> 9) 2^-23 (exponent bits spliced in) minus 1 - 2^-24: the result
// is exactly representable, so the subtraction is exact.
__device__ __forceinline__ float gumbel_e(uint32_t klo, uint32_t khi, uint32_t v) {
  const uint32_t h = elem_hash(klo, khi, v);
  const float f = __uint_as_float(__builtin_amdgcn_alignbit(0x7Fu, h, 9u));   // 0x3F800000 | h >> 9
  return -fast_log2(f - (1.0f - 0x1.0p-24f));
}


// ---------------------------------------------------------------------------
// Merge rules (deterministic: fixed order, lowest index wins ties).
// ---------------------------------------------------------------------------
struct SoftmaxState {
  float m;   // running max of y2 (base-2 scaled logits)
  float s;   // sum of exp2(y2 - m)
};

__device__ __forceinline__ void softmax_merge(float& m, float& s, float m2, float s2) {
  float mn = fmaxf(m, m2);
  float a = (m == mn) ? s : s * fast_exp2(m - mn);
  float b = (m2 == mn) ? s2 : s2 * fast_exp2(m2 - mn);
  m = mn;
  s = a + b;
}

// (key, index) packed into 64 bits so that unsigned order is the winner
// order: larger key first (the float's bits mapped to an order-preserving
// integer; -0 folded into +0), then lower index.  0 is below every pair.
__device__ __forceinline__ unsigned long long pack_best(float key, int idx) {
  uint32_t u = __float_as_uint(key + 0.0f);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)u << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)idx);
}

__device__ __forceinline__ int best_index(unsigned long long packed) {
  return (int)(0xFFFFFFFFu - (uint32_t)packed);
}

// true if (k2, i2) beats (k1, i1): larger key, or equal key and lower index.
__device__ __forceinline__ bool key_beats(float k2, int i2, float k1, int i1) {
  return (k2 > k1) || (k2 == k1 && i2 < i1);
}

template <typename T>
__device__ __forceinline__ T shfl_xor(T v, int m) {
  return __shfl_xor(v, m, 64);
}

// A chunk's draft partial: log-sum-exp state, the leader's key and index, and
// the tempered logit y at the leader (sampling; greedy: z).
struct DraftPart {
  float m, s, key, zb;
  int idx;
};

__device__ __forceinline__ void part_merge(DraftPart& a, const DraftPart& b) {
  softmax_merge(a.m, a.s, b.m, b.s);
  if (key_beats(b.key, b.idx, a.key, a.idx)) {
    a.key = b.key;
    a.idx = b.idx;
    a.zb = b.zb;
  }
}

__device__ __forceinline__ DraftPart part_shfl(const DraftPart& p, int mask) {
  return DraftPart{shfl_xor(p.m, mask), shfl_xor(p.s, mask), shfl_xor(p.key, mask), shfl_xor(p.zb, mask),
                   shfl_xor(p.idx, mask)};
}

__device__ __forceinline__ bf16x8_t load_bf16x8(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8_t*>(p);
}

__device__ __forceinline__ bf16x8_t zero_bf16x8() {
  bf16x8_t z;
#pragma unroll
  for (int i = 0; i < 8; ++i) z[i] = (__bf16)0.0f;
  return z;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

}  // namespace dspark
