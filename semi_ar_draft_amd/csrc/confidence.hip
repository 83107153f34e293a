// Confidence head with per-position temperature scaling, and survival
// products.
//
// [blog] "置信度头：预测自己的命运": c_k = sigmoid of a linear map of
// [h_k ; emb(x_{k-1})]; [blog] "校准问题：原始置信度不可靠": per-position
// temperature T_k applied to the logit; [teardown] "硬件感知前缀调度器" and
// [summary] section 4: survival a_j = prod_{i<=j} c_i.
//
// The head is a GEMV over 2 x 4096 bf16 values per (request, position): it is
// bound by HBM (h and the gathered embedding rows), so each (b, k) row gets
// one 256-thread workgroup streaming 16-byte loads with fp32 accumulation.
#include "common.hpp"
#include "internal.hpp"

namespace dspark {
namespace {

constexpr int kConfThreads = 256;

__device__ __forceinline__ float dot8(const uint16_t* x, const uint16_t* w) {
  const uint4 xv = *reinterpret_cast<const uint4*>(x);
  const uint4 wv = *reinterpret_cast<const uint4*>(w);
  const uint32_t xs[4] = {xv.x, xv.y, xv.z, xv.w};
  const uint32_t ws[4] = {wv.x, wv.y, wv.z, wv.w};
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float x0 = __uint_as_float(xs[i] << 16), x1 = __uint_as_float(xs[i] & 0xFFFF0000u);
    const float w0 = __uint_as_float(ws[i] << 16), w1 = __uint_as_float(ws[i] & 0xFFFF0000u);
    acc = __builtin_fmaf(x0, w0, acc);
    acc = __builtin_fmaf(x1, w1, acc);
  }
  return acc;
}

__global__ __launch_bounds__(kConfThreads) void confidence_impl(const ConfArgs a) {
  const int row = blockIdx.x;           // b * gamma + (k - 1)
  const int b = row / a.gamma;
  const int k = row % a.gamma + 1;
  int prev = (k == 1) ? a.anchor[b] : a.tokens[(int64_t)b * a.gamma + k - 2];
  if ((unsigned)prev >= (unsigned)a.V) {
    if (threadIdx.x == 0) atomicOr(a.err, kErrToken);
    prev = 0;
  }
  const uint16_t* h = a.h + (int64_t)row * a.dh;
  const uint16_t* e = a.E + (int64_t)prev * a.de;
  float acc = 0.f;
  for (int i = threadIdx.x; i < (a.dh >> 3); i += kConfThreads) acc += dot8(h + 8 * i, a.wc + 8 * i);
  for (int i = threadIdx.x; i < (a.de >> 3); i += kConfThreads)
    acc += dot8(e + 8 * i, a.wc + a.dh + 8 * i);
#pragma unroll
  for (int mask = 1; mask < 64; mask <<= 1) acc += shfl_xor(acc, mask);
  __shared__ float red[kConfThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    float l = red[0];
#pragma unroll
    for (int w = 1; w < kConfThreads / 64; ++w) l += red[w];
    l += a.bc;
    const float T = a.sts ? a.sts[k - 1] : 1.0f;
    const float c = 1.0f / (1.0f + __expf(-l / T));
    a.conf[row] = c;
  }
}

__global__ __launch_bounds__(256) void survival_impl(const ConfArgs a) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= a.B) return;
  float s = 1.0f;
  for (int k = 0; k < a.gamma; ++k) {
    s *= a.conf[(int64_t)b * a.gamma + k];
    a.surv[(int64_t)b * a.gamma + k] = s;
  }
}

}  // namespace

const void* confidence_kernel() { return (const void*)&confidence_impl; }
const void* survival_kernel() { return (const void*)&survival_impl; }

}  // namespace dspark
