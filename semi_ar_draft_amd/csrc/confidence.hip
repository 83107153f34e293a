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

__global__ __launch_bounds__(kConfThreads) void confidence_impl(const ConfArgs a) {
  const int b = blockIdx.x;
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
      int prev = (k == 1) ? a.anchor[b] : a.tokens[(int64_t)b * a.gamma + k - 2];
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

}  // namespace

const void* confidence_kernel() { return (const void*)&confidence_impl; }

}  // namespace dspark
