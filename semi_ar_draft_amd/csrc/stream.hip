// Streaming-read calibration, not part of the decoding path: the sum of n
// floats, each read once from memory in 16-byte loads.  Timed over a buffer
// larger than the last-level cache it measures what a plain read reaches on
// this part: the practical ceiling the path's streaming kernels are compared
// with.  Each workgroup reads one contiguous block, sixteen 4 KB pieces per
// iteration, with non-temporal loads (data read once should not displace
// what the caches hold): on this part that reads about 15% faster than a
// grid-stride loop of ordinary loads.
#include "common.hpp"
#include "internal.hpp"

namespace dspark {
namespace {

constexpr int kUnroll = 16;

__device__ __forceinline__ float4 load_nt(const float4* p) {
  const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
  return make_float4(v[0], v[1], v[2], v[3]);
}

// Workgroup w sums float4 indices [w per, (w + 1) per) into partials[w];
// workgroup 0 also adds the n % 4 trailing floats.
__global__ __launch_bounds__(kStreamThreads) void stream_read_impl(const StreamArgs a) {
  const float4* __restrict__ x = reinterpret_cast<const float4*>(a.x);
  const int64_t per = (a.n4 + gridDim.x - 1) / gridDim.x;
  const int64_t b0 = (int64_t)blockIdx.x * per;
  const int64_t b1 = b0 + per < a.n4 ? b0 + per : a.n4;
  int64_t i = b0 + threadIdx.x;
  float acc = 0.0f;
  for (; i + (kUnroll - 1) * kStreamThreads < b1; i += kUnroll * kStreamThreads) {
    float4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = load_nt(x + i + u * kStreamThreads);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc += (v[u].x + v[u].y) + (v[u].z + v[u].w);
  }
  for (; i < b1; i += kStreamThreads) {
    const float4 v = load_nt(x + i);
    acc += (v.x + v.y) + (v.z + v.w);
  }
  if (blockIdx.x == 0 && (int64_t)threadIdx.x < a.n - 4 * a.n4) acc += a.x[4 * a.n4 + threadIdx.x];
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) acc += shfl_xor(acc, m);
  __shared__ float red[kStreamThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) a.partials[blockIdx.x] = (red[0] + red[1]) + (red[2] + red[3]);
}

// One workgroup: the partials in a fixed order (thread t takes t, t + 256,
// ..., then a fixed tree).
__global__ __launch_bounds__(kStreamThreads) void stream_sum_impl(const StreamArgs a) {
  float acc = 0.0f;
  for (int i = threadIdx.x; i < a.n_part; i += kStreamThreads) acc += a.partials[i];
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) acc += shfl_xor(acc, m);
  __shared__ float red[kStreamThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) a.out[0] = (red[0] + red[1]) + (red[2] + red[3]);
}

}  // namespace

const void* stream_read_kernel() { return (const void*)&stream_read_impl; }
const void* stream_sum_kernel() { return (const void*)&stream_sum_impl; }

}  // namespace dspark
