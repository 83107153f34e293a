// Hardware-aware prefix scheduler: greedy admission with early stop.  The
// candidates are ranked by a kernel spread over the chip, then one workgroup
// scans the sorted list, finds the stop and counts K_b.
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

__device__ __forceinline__ uint64_t sched_key(float v, int i) {
  v = (v > 0.0f) ? v : 0.0f;        // NaN, negatives and -0 read as +0
  return ((uint64_t)(~__float_as_uint(v)) << 32) | (uint32_t)i;
}

// Sorting by ranking, spread over the whole chip: a sort inside the
// scheduler's single workgroup is one CU's work (a bitonic network over 4096
// keys took ~30 us).  Workgroup (g, set) ranks keys 16 g .. 16 g + 15 of
// the set against all n keys (the keys are distinct: the index is their low
// word): thread t compares key t % 16 with every 64th key, the counts merge
// by shuffles and across waves, and the key is stored at its rank.  Set 0:
// the survivals the count is chosen from (the older ones under the
// asynchronous rule); set 1: the current survivals (asynchronous rule only).
constexpr int kRankKeys = 16;

__global__ __launch_bounds__(kSchedThreads) void sched_rank_impl(const SchedArgs a) {
  __shared__ uint64_t all[kSchedKeys];
  __shared__ int part[kSchedThreads / 64][kRankKeys];
  const int n = a.B * a.gamma;
  const int set = blockIdx.y;
  const float* src = (set == 0 && a.surv_hist) ? a.surv_hist : a.surv;
  for (int j = threadIdx.x; j < n; j += kSchedThreads) all[j] = sched_key(src[j], j);
  __syncthreads();
  const int ks = threadIdx.x % kRankKeys;
  const int jg = threadIdx.x / kRankKeys;
  const int i = blockIdx.x * kRankKeys + ks;
  const uint64_t ki = i < n ? all[i] : 0ull;
  int cnt = 0;
  for (int j = jg; j < n; j += kSchedThreads / kRankKeys) cnt += all[j] < ki ? 1 : 0;
  // lane = 16 (jg mod 4) + ks: the four j-groups of a wave differ in lane bits 4, 5
  cnt += __shfl_xor(cnt, 16, 64);
  cnt += __shfl_xor(cnt, 32, 64);
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  if (lane < kRankKeys) part[wid][lane] = cnt;
  __syncthreads();
  if ((int)threadIdx.x < kRankKeys && i < n) {
    int r = 0;
#pragma unroll
    for (int w = 0; w < kSchedThreads / 64; ++w) r += part[w][threadIdx.x];
    a.sorted[(size_t)set * kSchedKeys + r] = ki;
  }
}

// The ranked keys of one set into LDS, padded with the largest key.
__device__ __forceinline__ void load_sorted(uint64_t* keys, const uint64_t* sorted, int n, int n_pad) {
  for (int i = threadIdx.x; i < n_pad; i += kSchedThreads) keys[i] = i < n ? sorted[i] : ~0ull;
  __syncthreads();
}

// Exclusive prefix (float64) of this thread's segment of the sorted list.
__device__ double segment_prefix(const uint64_t* keys, double* wave_tot, int n, int p0, int seg) {
  const int tid = threadIdx.x;
  double part = 0.0;
  for (int e = 0; e < seg; ++e) {
    const int p = p0 + e;
    if (p < n) part += (double)key_value(keys[p]);
  }
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
  return wave_pre + excl;
}

// (Theta, n) pairs: larger Theta first, then smaller n.
__device__ __forceinline__ bool theta_beats(double t2, int n2, double t1, int n1) {
  return t2 > t1 || (t2 == t1 && n2 < n1);
}

// ASYNC = 0: the synchronous rule (admit in sorted order, stop at the first
// n with Theta_n <= Theta_{n-1}).  ASYNC = 1: the count n* is the first
// maximum of Theta_n over the sorted historical survivals (no early stop),
// and the admitted candidates are the top n* of the current survivals.
template <int ASYNC>
__global__ __launch_bounds__(kSchedThreads) void schedule_impl(const SchedArgs a) {
  __shared__ uint64_t keys[kSchedKeys];
  __shared__ double wave_tot[kSchedThreads / 64];
  __shared__ double wave_th[kSchedThreads / 64];
  __shared__ int wave_n[kSchedThreads / 64];
  __shared__ int first_stop;
  __shared__ int s_nsel;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wid = tid >> 6;
  const int n = a.B * a.gamma;
  int n_pad = 2;
  while (n_pad < n) n_pad <<= 1;
  if (tid == 0) first_stop = 0x7fffffff;
  load_sorted(keys, a.sorted, n, n_pad);
  // each thread: a contiguous segment of the sorted list
  const int seg = (n_pad >= kSchedThreads) ? n_pad / kSchedThreads : 1;
  const int p0 = tid * seg;
  double S = segment_prefix(keys, wave_tot, n, p0, seg);
  const double Bd = (double)a.B;
  const double theta0 = Bd * (double)a.sps[a.B - 1];
  const int n_max = min(n, a.n_sps - a.B);
  int bidx[kPerThread];
  double S_at[kPerThread];
  double best_th = -1.0;
  int best_n = 0x7fffffff;
  for (int e = 0; e < seg; ++e) {
    const int p = p0 + e;
    bidx[e] = -1;
    S_at[e] = 0.0;
    if (p >= n) continue;
    const uint64_t key = keys[p];
    const double S_prev = S;
    S = S + (double)key_value(key);
    S_at[e] = S;
    bidx[e] = (int)((uint32_t)key) / a.gamma;
    if (p < n_max) {
      const int N = a.B + p + 1;
      const double th = (Bd + S) * (double)a.sps[N - 1];
      if (ASYNC) {
        if (theta_beats(th, p + 1, best_th, best_n)) {
          best_th = th;
          best_n = p + 1;
        }
      } else {
        const double th_prev = (p == 0) ? theta0 : (Bd + S_prev) * (double)a.sps[N - 2];
        if (th <= th_prev) atomicMin(&first_stop, p);
      }
    }
  }
  if (ASYNC) {
    // argmax over n (n = 0 is Theta_0): within waves, then across them
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const double t2 = __shfl_xor(best_th, d, 64);
      const int n2 = __shfl_xor(best_n, d, 64);
      if (theta_beats(t2, n2, best_th, best_n)) {
        best_th = t2;
        best_n = n2;
      }
    }
    if (lane == 0) {
      wave_th[wid] = best_th;
      wave_n[wid] = best_n;
    }
    __syncthreads();
    if (tid == 0) {
      double bt = theta0;
      int bn = 0;
      for (int w = 0; w < kSchedThreads / 64; ++w)
        if (theta_beats(wave_th[w], wave_n[w], bt, bn)) {
          bt = wave_th[w];
          bn = wave_n[w];
        }
      s_nsel = bn;
      *a.theta = bt;
      *a.n_selected = bn;
    }
    __syncthreads();
    // rank the current survivals; the admitted set is their top n*
    load_sorted(keys, a.sorted + kSchedKeys, n, n_pad);
    for (int e = 0; e < seg; ++e) {
      const int p = p0 + e;
      bidx[e] = p < n ? (int)((uint32_t)keys[p]) / a.gamma : -1;
    }
  } else {
    __syncthreads();
    const int nsel = min(first_stop, n_max);
    // Theta at the admitted set
    if (nsel == 0) {
      if (tid == 0) *a.theta = theta0;
    } else {
      for (int e = 0; e < seg; ++e) {
        if (p0 + e == nsel - 1) *a.theta = (Bd + S_at[e]) * (double)a.sps[a.B + nsel - 1];
      }
    }
    if (tid == 0) {
      *a.n_selected = nsel;
      s_nsel = nsel;
    }
  }
  // K_b: count admitted candidates per request (reusing the key storage)
  __syncthreads();
  const int nsel = s_nsel;
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

const void* schedule_rank_kernel() { return (const void*)&sched_rank_impl; }

const void* schedule_kernel(int async) {
  return async ? (const void*)&schedule_impl<1> : (const void*)&schedule_impl<0>;
}

}  // namespace dspark
