// GRU (RNN) head recurrence: s_k = GRU(s_{k-1}, W1[x_k]).
//
// [blog] "RNN Head：长程依赖": the sequential head may keep a GRU-style state
// that starts from a learned s_0 and absorbs every token drafted so far; the
// bias of position k is s_{k-1} projected onto the vocabulary (the projection
// itself runs in the sweep, with the state as the MFMA B operand).  The cell
// is the textbook GRU in the usual gate order (reset, update, new):
//   r  = sigmoid(W_ir x + b_ir + W_hr s + b_hr)
//   z  = sigmoid(W_iz x + b_iz + W_hz s + b_hz)
//   n  = tanh(W_in x + b_in + r * (W_hn s + b_hn))
//   s' = (1 - z) * n + z * s
// with x = W1[x_k], the sampled token's rank-r row; fp32 state, bf16 weights,
// products on bf16 MFMA with fp32 accumulation (inputs split into hi + lo).
#include "common.hpp"
#include "internal.hpp"

namespace dspark {
namespace {

constexpr int kGruTile = 16;     // requests x hidden units per workgroup

__device__ __forceinline__ float sigmoid_f(float x) { return 1.0f / (1.0f + __expf(-x)); }
__device__ __forceinline__ float tanh_f(float x) { return 1.0f - 2.0f / (__expf(2.0f * x) + 1.0f); }

// s_0 for every request.
__global__ __launch_bounds__(256) void gru_init_impl(const GruArgs a) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)a.B * a.R) return;
  a.states[i] = bf16_to_f32(a.s0[i % a.R]);
}

// bf16x8 fragment from 8 consecutive fp32 values, split into hi + lo
// (hi = RNE(x), lo = RNE(x - hi)): a product with a bf16 weight then keeps
// x to about 2^-16 relative.
__device__ __forceinline__ void split8(const float* p, bf16x8_t& hi, bf16x8_t& lo) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const __bf16 h = (__bf16)v[i];
    hi[i] = h;
    lo[i] = (__bf16)(v[i] - (float)h);
  }
}

// One workgroup per 16 hidden units x 16 requests, kGruWaves(R) waves
// splitting the K (= r) dimension: wave w takes K steps w NS/KW ..
// (w+1) NS/KW - 1 of the six gate products (W_i{r,z,n} x and W_h{r,z,n} s,
// 16 x 16 x r MFMA tiles with the weight rows as the A operand and the
// request's input row / state as B, split into hi + lo bf16).  The partial
// products meet in LDS and wave 0 adds them in wave order; its lane l then
// holds units j0 + 4(l/16) + i of request b0 + l % 16 and applies the cell.
template <int R>
constexpr int gru_waves() { return R / 32 >= 4 ? 4 : R / 32; }

template <int R>
__global__ __launch_bounds__(64 * gru_waves<R>()) void gru_step_impl(const GruArgs a) {
  constexpr int NS = R / 32;
  constexpr int KW = gru_waves<R>();
  constexpr int SPW = NS / KW;           // K steps per wave
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int n = lane & 15;
  const int q = lane >> 4;
  const int j0 = blockIdx.x * kGruTile;
  const int b0 = blockIdx.y * kGruTile;
  const int b = b0 + n;
  const bool ok = b < a.B;
  const int bx = ok ? b : 0;
  // x_k of request b: the maximum over position k's slot groups (the four
  // lanes of a request read a quarter of the groups each)
  unsigned long long m = 0ull;
#pragma unroll
  for (int i = 0; i < kBestGroups / 4; ++i) {
    const unsigned long long v = a.best[(int64_t)(q * (kBestGroups / 4) + i) * a.B + bx];
    m = v > m ? v : m;
  }
#pragma unroll
  for (int sh = 16; sh <= 32; sh <<= 1) {
    const unsigned long long o = __shfl_xor(m, sh, 64);
    m = o > m ? o : m;
  }
  int tok = best_index(m);
  if ((unsigned)tok >= (unsigned)a.V) {
    if (ok && q == 0 && wid == 0) atomicOr(a.err, kErrToken);
    tok = 0;
  }
  const float* srow = a.states + (int64_t)(a.k - 1) * a.B * R + (int64_t)bx * R;
  bf16x8_t xh[SPW], xl[SPW], sh_[SPW], sl[SPW];
#pragma unroll
  for (int e = 0; e < SPW; ++e) {
    const int s = wid * SPW + e;
    if (a.w1_bf16) {
      xh[e] = load_bf16x8(static_cast<const uint16_t*>(a.W1) + (int64_t)tok * R + 32 * s + 8 * q);
      xl[e] = zero_bf16x8();
    } else {
      split8(static_cast<const float*>(a.W1) + (int64_t)tok * R + 32 * s + 8 * q, xh[e], xl[e]);
    }
    split8(srow + 32 * s + 8 * q, sh_[e], sl[e]);
  }
  f32x4_t gi[3], gh[3];
#pragma unroll
  for (int g = 0; g < 3; ++g) {
    gi[g] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    gh[g] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const uint16_t* wi = a.W_ih + (int64_t)(g * R + j0 + n) * R + 8 * q;
    const uint16_t* wh = a.W_hh + (int64_t)(g * R + j0 + n) * R + 8 * q;
#pragma unroll
    for (int e = 0; e < SPW; ++e) {
      const int s = wid * SPW + e;
      const bf16x8_t ai = load_bf16x8(wi + 32 * s);
      const bf16x8_t ah = load_bf16x8(wh + 32 * s);
      gi[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ai, xh[e], gi[g], 0, 0, 0);
      gi[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ai, xl[e], gi[g], 0, 0, 0);
      gh[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, sh_[e], gh[g], 0, 0, 0);
      gh[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, sl[e], gh[g], 0, 0, 0);
    }
  }
  if constexpr (KW > 1) {
    __shared__ float part[KW - 1][6][4][64];
    if (wid > 0) {
#pragma unroll
      for (int g = 0; g < 3; ++g)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          part[wid - 1][g][i][lane] = gi[g][i];
          part[wid - 1][3 + g][i][lane] = gh[g][i];
        }
    }
    __syncthreads();
    if (wid > 0) return;
#pragma unroll
    for (int w = 0; w < KW - 1; ++w)
#pragma unroll
      for (int g = 0; g < 3; ++g)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          gi[g][i] += part[w][g][i][lane];
          gh[g][i] += part[w][3 + g][i][lane];
        }
  }
  if (!ok) return;
  float* out = a.states + (int64_t)a.k * a.B * R + (int64_t)b * R;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int j = j0 + 4 * q + i;
    const float rg = sigmoid_f(gi[0][i] + bf16_to_f32(a.b_ih[j]) + gh[0][i] + bf16_to_f32(a.b_hh[j]));
    const float zg = sigmoid_f(gi[1][i] + bf16_to_f32(a.b_ih[R + j]) + gh[1][i] + bf16_to_f32(a.b_hh[R + j]));
    const float ng = tanh_f(gi[2][i] + bf16_to_f32(a.b_ih[2 * R + j]) +
                            rg * (gh[2][i] + bf16_to_f32(a.b_hh[2 * R + j])));
    out[j] = (1.0f - zg) * ng + zg * srow[j];
  }
}

}  // namespace

const void* gru_init_kernel() { return (const void*)&gru_init_impl; }
int gru_step_threads(int r) { return r >= 128 ? 256 : (r == 64 ? 128 : 64); }

const void* gru_step_kernel(int r) {
  switch (r) {
    case 32: return (const void*)&gru_step_impl<32>;
    case 64: return (const void*)&gru_step_impl<64>;
    case 128: return (const void*)&gru_step_impl<128>;
    case 256: return (const void*)&gru_step_impl<256>;
    default: return nullptr;
  }
}

}  // namespace dspark
