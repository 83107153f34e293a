// Hardware-aware prefix scheduler: greedy admission with early stop, in one
// workgroup.
//
// [blog] "硬件感知前缀调度器" steps 1-4: build every (request, length)
// candidate with its survival a, sort from high to low, admit greedily while
// tracking Theta = tau * SPS, stop once Theta stops increasing; [summary]
// section 4 (expected accepted tokens times the steps/s of the resulting
// batch, read from a profiled table).
//
// Greedy admission in sorted order makes the admitted set after n steps the
// top-n candidates, so every Theta_n is known once the sorted prefix sums
// S_n are: Theta_n = (B + S_n) * SPS[B + n - 1].  The sequential loop of the
// definition becomes sort -> scan -> first n with Theta_n <= Theta_{n-1}.
// Keys are 64-bit: (~bits(a)) << 32 | (b * gamma + j - 1), so an ascending
// sort orders a descending, then request, then position.  Sums and Theta are
// float64: sums of float32 survivals are exact in float64 for any realistic
// spread of magnitudes, so the order of the scan does not change them.
#include "common.hpp"
#include "internal.hpp"

namespace dspark {
namespace {

constexpr int kSchedKeys = 4096;   // B * gamma <= kSchedKeys
constexpr int kPerThread = kSchedKeys / kSchedThreads;

__device__ __forceinline__ float key_value(uint64_t k) {
  return __uint_as_float(~(uint32_t)(k >> 32));
}

__global__ __launch_bounds__(kSchedThreads) void schedule_impl(const SchedArgs a) {
  __shared__ uint64_t keys[kSchedKeys];
  __shared__ double wave_tot[kSchedThreads / 64];
  __shared__ int first_stop;
  const int tid = threadIdx.x;
  const int n = a.B * a.gamma;
  int n_pad = 2;
  while (n_pad < n) n_pad <<= 1;
  for (int i = tid; i < n_pad; i += kSchedThreads) {
    uint64_t key = ~0ull;
    if (i < n) {
      float v = a.surv[i];
      v = (v > 0.0f) ? v : 0.0f;    // NaN, negatives and -0 read as +0
      key = ((uint64_t)(~__float_as_uint(v)) << 32) | (uint32_t)i;
    }
    keys[i] = key;
  }
  if (tid == 0) first_stop = 0x7fffffff;
  __syncthreads();
  // bitonic sort, ascending
  for (int size = 2; size <= n_pad; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int t = tid; t < (n_pad >> 1); t += kSchedThreads) {
        const int i = 2 * t - (t & (stride - 1));
        const int jx = i + stride;
        const uint64_t ki = keys[i], kj = keys[jx];
        const bool up = (i & size) == 0;
        if ((ki > kj) == up) {
          keys[i] = kj;
          keys[jx] = ki;
        }
      }
      __syncthreads();
    }
  }
  // each thread: a contiguous segment of the sorted list
  const int seg = (n_pad >= kSchedThreads) ? n_pad / kSchedThreads : 1;
  const int p0 = tid * seg;
  double part = 0.0;
  for (int e = 0; e < seg; ++e) {
    const int p = p0 + e;
    if (p < n) part += (double)key_value(keys[p]);
  }
  // inclusive scan of the per-thread sums: within waves, then across waves
  const int lane = tid & 63, wid = tid >> 6;
  double inc = part;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const double o = __shfl_up(inc, d, 64);
    if (lane >= d) inc += o;
  }
  if (lane == 63) wave_tot[wid] = inc;
  __syncthreads();
  double wave_pre = 0.0;
  for (int w = 0; w < wid; ++w) wave_pre += wave_tot[w];
  double excl = __shfl_up(inc, 1, 64);
  if (lane == 0) excl = 0.0;
  double S = wave_pre + excl;           // exclusive prefix of this segment
  const double Bd = (double)a.B;
  const int n_max = min(n, a.n_sps - a.B);
  int bidx[kPerThread];
  double S_at[kPerThread];
  for (int e = 0; e < seg; ++e) {
    const int p = p0 + e;
    bidx[e] = -1;
    S_at[e] = 0.0;
    if (p >= n) continue;
    const uint64_t key = keys[p];
    const double av = (double)key_value(key);
    const double S_prev = S;
    S = S + av;
    S_at[e] = S;
    bidx[e] = (int)((uint32_t)key) / a.gamma;
    if (p < n_max) {
      const int N = a.B + p + 1;
      const double th = (Bd + S) * (double)a.sps[N - 1];
      const double th_prev = (p == 0) ? Bd * (double)a.sps[a.B - 1] : (Bd + S_prev) * (double)a.sps[N - 2];
      if (th <= th_prev) atomicMin(&first_stop, p);
    }
  }
  __syncthreads();
  const int nsel = min(first_stop, n_max);
  // Theta at the admitted set
  if (nsel == 0) {
    if (tid == 0) *a.theta = Bd * (double)a.sps[a.B - 1];
  } else {
    for (int e = 0; e < seg; ++e) {
      if (p0 + e == nsel - 1) *a.theta = (Bd + S_at[e]) * (double)a.sps[a.B + nsel - 1];
    }
  }
  if (tid == 0) *a.n_selected = nsel;
  // K_b: count admitted candidates per request (reusing the key storage)
  int* counts = reinterpret_cast<int*>(keys);
  __syncthreads();
  for (int i = tid; i < a.B; i += kSchedThreads) counts[i] = 0;
  __syncthreads();
  for (int e = 0; e < seg; ++e) {
    if (p0 + e < nsel) atomicAdd(&counts[bidx[e]], 1);
  }
  __syncthreads();
  for (int i = tid; i < a.B; i += kSchedThreads) a.K[i] = counts[i];
}

}  // namespace

const void* schedule_kernel() { return (const void*)&schedule_impl; }

}  // namespace dspark
