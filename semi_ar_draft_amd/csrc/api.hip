// C ABI of libdspark: context, argument checks, workspace, launch plans
// (per-position sweeps or, for small batches, the whole-draft kernel) and the
// HIP-graph cache of the sequential draft loop.
#include <dlfcn.h>
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "dspark.h"
#include "common.hpp"
#include "internal.hpp"

using namespace dspark;

// Scratch of the allocation-free draft entry point (dspark_draft_markov_static):
// chained-draft counters and release flags, the running-best slot groups and
// the chunk partials, at fixed offsets.  One copy per GPU the library runs
// on, held until the process ends; every call on that GPU shares it.
constexpr size_t kScratchChainOff = 0;                        // 65 counter words
constexpr size_t kScratchFlagsOff = 64 << 10;                 // kChainMaxGrid lines of 128 bytes
constexpr size_t kScratchBestOff = kScratchFlagsOff + (size_t)kChainMaxGrid * 128;
constexpr size_t kScratchBestBytes = 1 << 20;                 // B * gamma * 16 slots of 8 bytes
constexpr size_t kScratchPartOff = kScratchBestOff + kScratchBestBytes;
constexpr size_t kScratchBytes = 16u << 20;
constexpr size_t kScratchPartBytes = kScratchBytes - kScratchPartOff;
static_assert(kScratchPartOff % 256 == 0, "scratch regions stay 256-byte aligned");
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

// Device address of `scratch` on each device, taken once per device with that
// device current (the array's name is not a device address in host code).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
int g_scratch_rc[kMaxDevices] = {};        // 0: not yet taken, 1: ready, -1: failed

// Called from dspark_create with `device` current: the address, and the whole
// array cleared once (everything the calls expect at zero starts there; each
// call leaves it zero again).
void scratch_setup(int device) {
  if (device < 0 || device >= kMaxDevices) return;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_rc[device] != 0) return;
  void* p = nullptr;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p ||
      hipMemset(p, 0, kScratchBytes) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
    (void)hipGetLastError();
    g_scratch_rc[device] = -1;
    return;
  }
  g_scratch_ptr[device] = p;
  g_scratch_rc[device] = 1;
}

void* scratch_ptr(int device) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  return g_scratch_rc[device] == 1 ? g_scratch_ptr[device] : nullptr;
}

constexpr int kVersion = 101;

struct KernelNode {
  int cls;
  const void* fn;
  dim3 grid, block;
  // argument storage: the largest argument block
  alignas(16) unsigned char args[sizeof(SweepArgs) > sizeof(CombineArgs) ? sizeof(SweepArgs)
                                                                        : sizeof(CombineArgs)];
};

// Instantiated graph of one draft loop shape; node parameters are rewritten
// before each launch, so one graph serves every buffer set and seed.
struct DraftGraph {
  int B = 0, gamma = 0, V = 0, r = 0, wdtype = -1, mode = -1, grid = 0, n_vc = 0;
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  std::vector<hipGraphNode_t> nodes;
};

}  // namespace

struct dspark_ctx {
  int device = 0;
  int cu_count = 256;
  std::string err;
  void* ws = nullptr;
  size_t ws_bytes = 0;
  int32_t* dev_err = nullptr;
  bool use_graph = false;
  int sweep_waves_per_cu = 8;     // occupancy target of the vocabulary sweeps
  // whole-draft kernel (Markov head, bf16, r = 256): used up to persist_max_b
  // requests (at most 128), and whether the device runs cooperative launches
  // (-1 = not yet asked).  It keeps W2 in registers at one wave per SIMD; its
  // fold is then issue-bound, so it wins only while the batch is small
  // (measured draft calls against the per-position sweeps: 1.5x faster at
  // B = 16, 1.3x at 32, 1.1x at 40-48, even at 56-64, 0.75x at 128).
  int persist_max_b = 48;
  int coop = -1;
  // launch it cooperatively (co-residency guaranteed by the runtime, also
  // under concurrent kernels; ~20-25 us more per call here); false: a plain
  // launch of one workgroup per CU, for callers that own an idle device
  bool persist_coop = true;
  // cooperative launches the runtime refused (each such call ran on the
  // per-position sweeps instead)
  long coop_refused = 0;
  int bar_test = 0;               // failure injection (tests): barriers time out
  unsigned int* bar = nullptr;    // its grid barrier counter (inside dev_err's block)
  // chained draft kernel (Markov head, bf16, r in {128, 256}, one request quad
  // of three or four 32-row groups): every position in one launch; its ticket
  // and per-position counters (inside dev_err's block, 33 words)
  bool use_chain = true;
  unsigned int* chain = nullptr;  // 65 words: tickets, then per-position counters from word 32
  unsigned int* chain_flags = nullptr;   // one 128-byte line per workgroup (kChainMaxGrid)
  int chain_wg_per_cu = -1;       // resident workgroups per CU (-1 = not yet asked)
  // shape of the chained draft: waves per workgroup, request rows per wave
  // (a request group is their product; two groups of 64 would interleave
  // their chains), ring steps loaded ahead, and vocabulary chunks per
  // position (0: one per resident workgroup).  Measured draft calls
  // (sampling, B = 128, gamma = 7, V = 151936): 8 waves x 16 rows, two steps
  // ahead, one 8-wave workgroup and one chunk per CU 207-209 us; three or
  // four steps ahead 215-217; 512 or 384 chunks 263-284 (a workgroup's
  // second item of a position repeats the set-up); two 4-wave workgroups
  // per CU with 32 rows per wave 216-224 (the two workgroups of a CU finish
  // their items several us apart); two groups of 64 requests with 16 rows
  // per wave 250 (W2 streamed twice per position).
  int chain_waves = 8, chain_rows = 16, chain_depth = 2, chain_chunks = 0;
  // shared-tile sweeps: 16-wide tiles per ring step and steps loaded ahead
  int draft_nt = 2, draft_depth = 1;
  // the GRU head's sweep holds its state as hi + lo fragments, so its
  // two-tile steps fold tile by tile (236 VGPRs: two waves per SIMD; a
  // two-tile fold needed 268)
  int gru_nt = 2, gru_depth = 1;
  int resid_nt = 1, resid_depth = 1;
  // temperature fit: scoring workgroups per CU (each flushes its n_bins x
  // n_grid sums into the global ones with 64-bit atomics).  Measured at 2^20
  // drafts, 64 candidates, 15 bins, us per position: 1024-thread workgroups
  // 37.6 / 34.9 at 1 / 2 per CU; 512-thread 42.9 / 38.5 / 39.5 at 1 / 2 / 3;
  // 256-thread 57 / 44 / 40 / 45 / 49 / 54 at 1 / 2 / 4 / 5 / 6 / 8.
  int sts_wg_per_cu = 2;
  // its (bin, candidate) sums and finished-workgroup counter, zero between
  // passes (allocated zeroed at the first fit)
  unsigned long long* sts_buf = nullptr;
  // verify: last target row of each window but the final one (window k covers
  // rows verify_win[k-1]+1 .. verify_win[k]); 0 ends the list.  Rows 1-2,
  // 3-4, then 5..K_b+1: measured steps on the headline batch (gamma 7, mean
  // acceptance 0.62), two boxes, alternating runs: 342.4 us against 342.7
  // for {1-2, 3-5, 6-8}, 345.2 for {1-2, 3, 4-8}, 346.8 for {1-2, 3-4, 5-6,
  // 7-8}; on another box 355.0 against 358.0 for {1-2, 3, 4-8}, 358.5 for
  // {1, 2-3, 4-8}, 362 for {1-2, 3-8} and {1-2, 3, 4, 5-8} (each window costs
  // a row pass and a decision launch; a wider window reads rows that are not
  // needed)
  int verify_win[8] = {2, 4, 0, 0, 0, 0, 0, 0};
  // later windows walk a list of the pending requests (else one workgroup per
  // row chunk of every request, most of which find it decided)
  bool verify_list = true;
  // verify chain: every needed target row of the call in one launch, each
  // request's rows decided one after another inside it (DSPARK_VERIFY_CHAIN);
  // its counter block (zero between calls) and resident workgroups per CU
  bool verify_chain = false;
  unsigned int* vq = nullptr;
  size_t vq_n = 0;
  int vchain_wg_per_cu = 0;
  int vchain_wg = 0;              // workgroups per CU of its grid (0: as many as are resident)
  int vchain_ahead = 2;           // rows of a request read ahead of its decisions
  // per-request counters of dspark_draft_markov_conf (zero between calls)
  unsigned int* cm_cnt = nullptr;
  size_t cm_n = 0;
  // draft: running best (key, index) per (position, request), zero between calls
  unsigned long long* best = nullptr;
  size_t best_n = 0;
  std::vector<DraftGraph> graphs;
  // kernel timing (benchmarks): event pairs around every launch while enabled
  bool timing = false;
  struct Pending {
    int cls;
    hipEvent_t a, b;
  };
  std::vector<hipEvent_t> ev_free;
  std::vector<Pending> pending;
};

namespace {

int fail(dspark_ctx* c, int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  if (c) c->err = buf;
  return code;
}

#define DSPARK_HIP(c, call)                                                             \
  do {                                                                                  \
    hipError_t e_ = (call);                                                             \
    if (e_ != hipSuccess)                                                               \
      return fail((c), DSPARK_EHIP, "%s failed: %s", #call, hipGetErrorString(e_));     \
  } while (0)

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

struct DeviceGuard {
  int prev = -1;
  bool ok = true;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    if (prev != dev) ok = hipSetDevice(dev) == hipSuccess;
  }
  ~DeviceGuard() {
    if (prev >= 0) (void)hipSetDevice(prev);
  }
};

// Grow the workspace to at least `bytes`.  Growing waits for the device so
// that no enqueued kernel still uses the old buffer.
int ensure_ws(dspark_ctx* c, size_t bytes) {
  if (bytes <= c->ws_bytes) return DSPARK_OK;
  DSPARK_HIP(c, hipDeviceSynchronize());
  if (c->ws) (void)hipFree(c->ws);
  c->ws = nullptr;
  c->ws_bytes = 0;
  size_t want = bytes + bytes / 4;
  if (hipMalloc(&c->ws, want) != hipSuccess) {
    (void)hipGetLastError();
    return fail(c, DSPARK_ENOMEM, "workspace allocation of %zu bytes failed", want);
  }
  c->ws_bytes = want;
  return DSPARK_OK;
}

// The draft's running bests must be zero when a call starts; every call
// clears the ones it used, so they are zeroed only when (re)allocated.
int ensure_best(dspark_ctx* c, size_t n) {
  if (n <= c->best_n) return DSPARK_OK;
  DSPARK_HIP(c, hipDeviceSynchronize());
  if (c->best) (void)hipFree(c->best);
  c->best = nullptr;
  c->best_n = 0;
  if (hipMalloc(&c->best, n * sizeof(unsigned long long)) != hipSuccess) {
    (void)hipGetLastError();
    return fail(c, DSPARK_ENOMEM, "allocation of %zu bytes failed", n * sizeof(unsigned long long));
  }
  DSPARK_HIP(c, hipMemset(c->best, 0, n * sizeof(unsigned long long)));
  c->best_n = n;
  return DSPARK_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Verify counters (B task counters, then the decided-request counter on its
// own line): zeroed when (re)allocated; every call leaves them zero.
int ensure_cm(dspark_ctx* c, size_t n) {
  if (n <= c->cm_n) return DSPARK_OK;
  DSPARK_HIP(c, hipDeviceSynchronize());
  if (c->cm_cnt) (void)hipFree(c->cm_cnt);
  c->cm_cnt = nullptr;
  c->cm_n = 0;
  const size_t m = std::max<size_t>(n, 1024);
  if (hipMalloc(&c->cm_cnt, m * sizeof(unsigned int)) != hipSuccess) {
    (void)hipGetLastError();
    return fail(c, DSPARK_ENOMEM, "allocation of %zu bytes failed", m * sizeof(unsigned int));
  }
  DSPARK_HIP(c, hipMemset(c->cm_cnt, 0, m * sizeof(unsigned int)));
  DSPARK_HIP(c, hipDeviceSynchronize());
  c->cm_n = m;
  return DSPARK_OK;
}

int ensure_vq(dspark_ctx* c, size_t words) {
  if (words <= c->vq_n) return DSPARK_OK;
  DSPARK_HIP(c, hipDeviceSynchronize());
  if (c->vq) (void)hipFree(c->vq);
  c->vq = nullptr;
  c->vq_n = 0;
  if (hipMalloc(&c->vq, words * sizeof(unsigned int)) != hipSuccess) {
    (void)hipGetLastError();
    return fail(c, DSPARK_ENOMEM, "allocation of %zu bytes failed", words * sizeof(unsigned int));
  }
  DSPARK_HIP(c, hipMemset(c->vq, 0, words * sizeof(unsigned int)));
  DSPARK_HIP(c, hipDeviceSynchronize());
  c->vq_n = words;
  return DSPARK_OK;
}

// Vocabulary-sweep plan: aim at eight waves per CU, at least four 16-wide
// tiles per wave, and a grid that is a multiple of the XCD count.
struct SweepPlan {
  int n_rg, n_vc, n_tiles, grid;
  bool shared;
};

// Batches of three or more 32-row groups share each W2 tile across the four
// waves of a workgroup (bf16, r >= 128); smaller batches give every wave its
// own vocabulary chunk.
SweepPlan plan_sweep(const dspark_ctx* c, int B, int V, int r, int wdtype) {
  SweepPlan p;
  p.n_rg = (B + kRowsPerWave - 1) / kRowsPerWave;
  p.n_tiles = V / kTileV;
  p.shared = wdtype == DSPARK_BF16 && (r == 128 || r == 256) && p.n_rg >= 3;
  const int target_waves = c->sweep_waves_per_cu * c->cu_count;
  const int max_vc = p.n_tiles / 4 > 0 ? p.n_tiles / 4 : 1;
  long grid;
  if (p.shared) {
    const int n_rq = (p.n_rg + kWavesPerBlock - 1) / kWavesPerBlock;
    int n_vc = target_waves / (kWavesPerBlock * n_rq);
    if (n_vc > max_vc) n_vc = max_vc;
    if (n_vc < 1) n_vc = 1;
    p.n_vc = n_vc;
    grid = (long)n_rq * n_vc;
  } else {
    int n_vc = target_waves / p.n_rg;
    if (n_vc > max_vc) n_vc = max_vc;
    if (n_vc < 1) n_vc = 1;
    p.n_vc = n_vc;
    const long waves = (long)p.n_rg * p.n_vc;
    grid = (waves + kWavesPerBlock - 1) / kWavesPerBlock;
  }
  grid = (grid + 7) / 8 * 8;
  p.grid = (int)grid;
  return p;
}

int check_stream_rows(dspark_ctx* c, const char* name, const float* p, int64_t sb, int64_t sk, int B, int rows,
                      int V) {
  if (!p) return fail(c, DSPARK_EINVAL, "%s is NULL", name);
  if (!aligned16(p)) return fail(c, DSPARK_EINVAL, "%s must be 16-byte aligned", name);
  if ((sb & 3) || (sk & 3) || sb <= 0 || sk <= 0)
    return fail(c, DSPARK_EINVAL, "%s strides must be positive multiples of 4", name);
  // rows (b, k) must not overlap: request-major ([B][rows][V]-like) or
  // position-major ([rows][B][V]-like) placements
  const bool req_major = sk >= V && sb >= (int64_t)rows * sk;
  const bool pos_major = sb >= V && sk >= (int64_t)B * sb;
  if (!req_major && !pos_major)
    return fail(c, DSPARK_EINVAL, "%s strides (%lld, %lld) overlap rows of %d values", name, (long long)sb,
                (long long)sk, V);
  return DSPARK_OK;
}

int check_markov_shape(dspark_ctx* c, int B, int gamma, int V, int r, int wdtype, float T) {
  if (B < 1) return fail(c, DSPARK_EINVAL, "B must be >= 1 (got %d)", B);
  if (gamma < 1 || gamma > kMaxGamma) return fail(c, DSPARK_EINVAL, "gamma must be in 1..%d", kMaxGamma);
  if (V < kTileV || V % kTileV) return fail(c, DSPARK_EINVAL, "V must be a positive multiple of 16");
  if (wdtype != DSPARK_F32 && wdtype != DSPARK_BF16) return fail(c, DSPARK_EINVAL, "unknown weight dtype");
  if (!sweep_kernel(wdtype, r, kModeDraftGreedy, 0, 1, 0))
    return fail(c, DSPARK_EINVAL, "r must be one of 32, 64, 128, 256 (got %d)", r);
  if (!(T >= 0.0f) || !std::isfinite(T)) return fail(c, DSPARK_EINVAL, "temperature must be finite and >= 0");
  return DSPARK_OK;
}

hipError_t launch(const void* fn, dim3 grid, dim3 block, void* arg, hipStream_t s) {
  void* params[] = {arg};
  return hipLaunchKernel(fn, grid, block, params, 0, s);
}

hipError_t take_event(dspark_ctx* c, hipEvent_t* e) {
  if (!c->ev_free.empty()) {
    *e = c->ev_free.back();
    c->ev_free.pop_back();
    return hipSuccess;
  }
  return hipEventCreate(e);
}

// Cooperative launch (every workgroup resident at once); while timing is
// enabled it is bracketed by stream events (no dispatch-attached events for
// this launch type), which include the queue's ordering gap before it.
// A launch the runtime refuses (e.g. while another process holds the
// device's cooperative-launch resource) returns kCoopRefused with nothing
// of the kernel enqueued and the HIP error cleared; the caller takes
// another path.
constexpr int kCoopRefused = -1;

int klaunch_coop(dspark_ctx* c, int cls, const void* fn, dim3 grid, dim3 block, void* arg, hipStream_t s) {
  void* params[] = {arg};
  if (!c->timing) {
    if (hipLaunchCooperativeKernel(fn, grid, block, params, 0, s) != hipSuccess) {
      (void)hipGetLastError();
      return kCoopRefused;
    }
    return DSPARK_OK;
  }
  hipEvent_t a, b;
  DSPARK_HIP(c, take_event(c, &a));
  DSPARK_HIP(c, take_event(c, &b));
  DSPARK_HIP(c, hipEventRecord(a, s));
  if (hipLaunchCooperativeKernel(fn, grid, block, params, 0, s) != hipSuccess) {
    (void)hipGetLastError();
    c->ev_free.push_back(a);                             // recorded, never read: reusable
    c->ev_free.push_back(b);
    return kCoopRefused;
  }
  DSPARK_HIP(c, hipEventRecord(b, s));
  c->pending.push_back({cls, a, b});
  return DSPARK_OK;
}

// Launch one kernel; while timing is enabled, bracket it with events.
int klaunch(dspark_ctx* c, int cls, const void* fn, dim3 grid, dim3 block, void* arg, hipStream_t s) {
  if (!c->timing) {
    DSPARK_HIP(c, launch(fn, grid, block, arg, s));
    return DSPARK_OK;
  }
  // events attached to the dispatch itself: they bracket the kernel's
  // execution, not the queue's stream-ordering gap before it
  hipEvent_t a, b;
  DSPARK_HIP(c, take_event(c, &a));
  DSPARK_HIP(c, take_event(c, &b));
  void* params[] = {arg};
  DSPARK_HIP(c, hipExtLaunchKernel(fn, grid, block, params, 0, s, a, b, 0));
  c->pending.push_back({cls, a, b});
  return DSPARK_OK;
}

template <typename A>
void set_node(KernelNode& n, int cls, const void* fn, dim3 grid, dim3 block, const A& a) {
  static_assert(sizeof(A) <= sizeof(n.args), "argument block too large");
  n.cls = cls;
  n.fn = fn;
  n.grid = grid;
  n.block = block;
  memcpy(n.args, &a, sizeof(A));
}

hipKernelNodeParams node_params(KernelNode& n, void** holder) {
  hipKernelNodeParams p;
  memset(&p, 0, sizeof(p));
  p.func = const_cast<void*>(n.fn);
  p.gridDim = n.grid;
  p.blockDim = n.block;
  p.sharedMemBytes = 0;
  holder[0] = n.args;
  p.kernelParams = holder;
  p.extra = nullptr;
  return p;
}

// Launch kernel nodes one after the other with no events and no graph (the
// allocation-free path: nothing is created).
int run_direct(dspark_ctx* c, hipStream_t stream, std::vector<KernelNode>& nodes) {
  for (auto& n : nodes) DSPARK_HIP(c, launch(n.fn, n.grid, n.block, n.args, stream));
  return DSPARK_OK;
}

// Run a chain of kernel nodes on `stream`, through a cached graph when
// enabled.
int run_chain(dspark_ctx* c, hipStream_t stream, std::vector<KernelNode>& nodes, int B, int gamma, int V,
              int r, int wdtype, int mode, int grid, int n_vc) {
  if (!c->use_graph || c->timing) {
    for (auto& n : nodes) {
      const int rc = klaunch(c, n.cls, n.fn, n.grid, n.block, n.args, stream);
      if (rc) return rc;
    }
    return DSPARK_OK;
  }
  DraftGraph* g = nullptr;
  for (auto& x : c->graphs)
    if (x.B == B && x.gamma == gamma && x.V == V && x.r == r && x.wdtype == wdtype && x.mode == mode &&
        x.grid == grid && x.n_vc == n_vc && x.nodes.size() == nodes.size())
      g = &x;
  if (!g) {
    DraftGraph ng;
    ng.B = B;
    ng.gamma = gamma;
    ng.V = V;
    ng.r = r;
    ng.wdtype = wdtype;
    ng.mode = mode;
    ng.grid = grid;
    ng.n_vc = n_vc;
    DSPARK_HIP(c, hipGraphCreate(&ng.graph, 0));
    hipGraphNode_t prev = nullptr;
    for (auto& n : nodes) {
      void* holder[1];
      hipKernelNodeParams p = node_params(n, holder);
      hipGraphNode_t node;
      hipError_t e = hipGraphAddKernelNode(&node, ng.graph, prev ? &prev : nullptr, prev ? 1 : 0, &p);
      if (e != hipSuccess) {
        (void)hipGraphDestroy(ng.graph);
        return fail(c, DSPARK_EHIP, "hipGraphAddKernelNode failed: %s", hipGetErrorString(e));
      }
      ng.nodes.push_back(node);
      prev = node;
    }
    hipError_t e = hipGraphInstantiate(&ng.exec, ng.graph, nullptr, nullptr, 0);
    if (e != hipSuccess) {
      (void)hipGraphDestroy(ng.graph);
      return fail(c, DSPARK_EHIP, "hipGraphInstantiate failed: %s", hipGetErrorString(e));
    }
    c->graphs.push_back(std::move(ng));
    g = &c->graphs.back();
  } else {
    for (size_t i = 0; i < nodes.size(); ++i) {
      void* holder[1];
      hipKernelNodeParams p = node_params(nodes[i], holder);
      DSPARK_HIP(c, hipGraphExecKernelNodeSetParams(g->exec, g->nodes[i], &p));
    }
  }
  DSPARK_HIP(c, hipGraphLaunch(g->exec, stream));
  return DSPARK_OK;
}

// Whole-draft kernel eligibility: Markov head, bf16 weights, r = 256, a batch
// within persist_max_b (<= 128), a vocabulary the waves' register tiles
// cover, and room for one such workgroup per CU (its LDS and registers
// admit no second one, so a grid of one workgroup per CU is resident at once
// on an otherwise idle device; with persist_coop the device must also
// support cooperative launches).
bool use_persist(dspark_ctx* c, int B, int V, int r, int wdtype) {
  if (wdtype != DSPARK_BF16 || r != 256 || B > c->persist_max_b || B > 128) return false;
  if ((long)(V / kTileV) > (long)kPersistTiles * kWavesPerBlock * c->cu_count) return false;
  if (c->coop < 0) {
    int v = 1;
    if (c->persist_coop &&
        hipDeviceGetAttribute(&v, hipDeviceAttributeCooperativeLaunch, c->device) != hipSuccess) {
      (void)hipGetLastError();
      v = 0;
    }
    int ok = v;
    for (int m = kModeDraftGreedy; ok && m <= kModeDraftSample; ++m) {
      int nb = 0;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, draft_persist_kernel(m), 256, 0) != hipSuccess) {
        (void)hipGetLastError();
        nb = 0;
      }
      ok = nb >= 1;
    }
    c->coop = ok ? 1 : 0;
  }
  return c->coop == 1;
}

// Chained draft eligibility: Markov head, bf16, r in {128, 256}, a batch of
// three or four 32-row groups (65..128 requests: one request quad, the
// shared-tile layout), and the kernel's ring shape.
const void* chain_kernel_for(const dspark_ctx* c, int B, int r, int wdtype, int mode) {
  if (!c->use_chain || c->chain_wg_per_cu < 1 || wdtype != DSPARK_BF16 || B < 65 || B > 128) return nullptr;
  return draft_chain_kernel(r, mode, c->chain_depth, 2, c->chain_rows, c->chain_waves);
}

// Where a draft call keeps its partials, slot groups and chained-draft
// counters: the context's workspace (grown on demand), or the static
// scratch (the allocation-free entry point: nothing allocated, kernels
// launched directly -- no graph, no timing events -- and no whole-draft
// kernel).
struct DraftMem {
  bool fixed = false;
  unsigned char* base = nullptr;
};

}  // namespace

// The draft loop of either head: gamma sweeps (+ gamma - 1 GRU updates and
// the s_0 fill for the GRU head), then one combine.  `gru` null = Markov.
int draft_chain(dspark_ctx* c, hipStream_t stream, int B, int gamma, int V, int r, dspark_dtype wdtype,
                const float* U, int64_t u_stride_b, int64_t u_stride_k, const void* W1, const void* W2,
                const int32_t* anchor, const GruArgs* gru, const uint32_t* req_ids, float temperature,
                uint64_t seed, int32_t* tokens, float* lse, float* ytok, float* states,
                const DraftMem& mem = DraftMem(), CombineArgs* merge_out = nullptr, bool allow_persist = true) {
  int rc = check_markov_shape(c, B, gamma, V, r, (int)wdtype, temperature);
  if (rc) return rc;
  if ((rc = check_stream_rows(c, "U", U, u_stride_b, u_stride_k, B, gamma, V))) return rc;
  if (!W1 || !W2 || !tokens || !lse || !ytok) return fail(c, DSPARK_EINVAL, "null pointer argument");
  if (!aligned16(W1) || !aligned16(W2)) return fail(c, DSPARK_EINVAL, "W1/W2 must be 16-byte aligned");
  DeviceGuard dg(c->device);
  if (!dg.ok) return fail(c, DSPARK_EHIP, "hipSetDevice failed");

  const bool greedy = temperature == 0.0f;
  const int mode = greedy ? kModeDraftGreedy : kModeDraftSample;
  const SweepPlan pl = plan_sweep(c, B, V, r, (int)wdtype);
  const bool persist = allow_persist && !gru && !mem.fixed && use_persist(c, B, V, r, (int)wdtype);
  const void* cfn = (gru || persist) ? nullptr : chain_kernel_for(c, B, r, (int)wdtype, mode);
  const int chain_vc = c->chain_chunks > 0 ? c->chain_chunks : c->chain_wg_per_cu * c->cu_count;
  const int n_vc = persist ? kWavesPerBlock * c->cu_count
                           : cfn ? std::max(1, std::min(chain_vc, (pl.n_tiles + 1) / 2)) : pl.n_vc;
  const size_t npos = (size_t)B * n_vc;                // partials of one position
  const size_t npart = npos * gamma;
  const size_t off_pi = align256(npart * sizeof(float4));
  const size_t part_bytes = off_pi + align256(npart * sizeof(int2));
  const size_t n_best = (size_t)B * gamma * kBestGroups;
  float4* pf;
  int2* pi;
  unsigned long long* best;
  unsigned int* chain_ctr = c->chain;
  unsigned int* chain_flags = c->chain_flags;
  if (mem.fixed) {
    if (part_bytes > kScratchPartBytes || n_best * sizeof(unsigned long long) > kScratchBestBytes)
      return fail(c, DSPARK_EINVAL,
                  "this draft needs %zu bytes of partials and %zu of slot groups; the allocation-free draft "
                  "holds at most %zu and %zu (a %zu-byte scratch per GPU)",
                  part_bytes, n_best * sizeof(unsigned long long), kScratchPartBytes, kScratchBestBytes,
                  kScratchBytes);
    pf = reinterpret_cast<float4*>(mem.base + kScratchPartOff);
    pi = reinterpret_cast<int2*>(mem.base + kScratchPartOff + off_pi);
    best = reinterpret_cast<unsigned long long*>(mem.base + kScratchBestOff);
    chain_ctr = reinterpret_cast<unsigned int*>(mem.base + kScratchChainOff);
    chain_flags = reinterpret_cast<unsigned int*>(mem.base + kScratchFlagsOff);
  } else {
    if ((rc = ensure_ws(c, part_bytes))) return rc;
    if ((rc = ensure_best(c, n_best))) return rc;
    pf = reinterpret_cast<float4*>(c->ws);
    pi = reinterpret_cast<int2*>(static_cast<char*>(c->ws) + off_pi);
    best = c->best;
  }

  SweepArgs sa;
  memset(&sa, 0, sizeof(sa));
  sa.B = B;
  sa.gamma = gamma;
  sa.V = V;
  sa.n_rg = pl.n_rg;
  sa.n_vc = n_vc;
  sa.n_tiles = pl.n_tiles;
  sa.xcd_remap = 1;
  sa.U = U;
  sa.usb = u_stride_b;
  sa.usk = u_stride_k;
  sa.W1 = W1;
  sa.W2 = W2;
  sa.anchor = anchor;
  sa.tokens = tokens;
  sa.req = req_ids;
  sa.invT = greedy ? 1.0f : 1.0f / temperature;
  sa.s2 = greedy ? kLog2e : kLog2e / temperature;
  sa.seed = seed;
  sa.pf = pf;
  sa.pi = pi;
  sa.err = c->dev_err;
  CombineArgs ca;
  memset(&ca, 0, sizeof(ca));
  ca.B = B;
  ca.gamma = gamma;
  ca.V = V;
  ca.n_vc = n_vc;
  ca.greedy = greedy;
  ca.invT = sa.invT;
  ca.pf = pf;
  ca.pi = pi;
  ca.best = best;
  ca.tokens = tokens;
  ca.lse = lse;
  ca.ytok = ytok;
  ca.err = c->dev_err;

  if (persist) {
    // every position in one launch of one workgroup per CU, then the merge
    // (which also resets the launch's barrier counter)
    sa.best = best;
    sa.bar = c->bar;
    sa.bar_test = c->bar_test;
    ca.bar = c->bar;
    rc = c->persist_coop
             ? klaunch_coop(c, DSPARK_K_DRAFT_SWEEP, draft_persist_kernel(mode), dim3(c->cu_count), dim3(256), &sa,
                            stream)
             : klaunch(c, DSPARK_K_DRAFT_SWEEP, draft_persist_kernel(mode), dim3(c->cu_count), dim3(256), &sa, stream);
    if (rc == kCoopRefused) {
      // cooperative launch refused, nothing enqueued: this call runs on the
      // per-position sweeps (the next call tries the whole-draft kernel again)
      ++c->coop_refused;
      return draft_chain(c, stream, B, gamma, V, r, wdtype, U, u_stride_b, u_stride_k, W1, W2, anchor, gru,
                         req_ids, temperature, seed, tokens, lse, ytok, states, mem, merge_out, false);
    }
    if (rc) return rc;
    if (merge_out) {                                     // the caller's next launch merges
      *merge_out = ca;
      return DSPARK_OK;
    }
    return klaunch(c, DSPARK_K_DRAFT_COMBINE, combine_draft_kernel(), dim3(B, gamma), dim3(256), &ca, stream);
  }
  if (cfn) {
    // every position in one launch of persistent workgroups, then the merge
    // (which also clears the launch's counters)
    sa.best = best;
    sa.chain = chain_ctr;
    sa.chain_flags = chain_flags;
    sa.bar_test = c->bar_test;
    ca.chain = chain_ctr;
    const int group_rows = c->chain_waves * c->chain_rows;
    const long items = (long)gamma * n_vc * ((B + group_rows - 1) / group_rows);
    const long resident = (long)c->chain_wg_per_cu * c->cu_count;
    const int grid = (int)std::min(std::min(items, resident), (long)kChainMaxGrid);
    std::vector<KernelNode> nodes(merge_out ? 1 : 2);
    set_node(nodes[0], DSPARK_K_DRAFT_CHAIN, cfn, dim3(grid), dim3(64 * c->chain_waves), sa);
    if (merge_out)
      *merge_out = ca;
    else
      set_node(nodes[1], DSPARK_K_DRAFT_COMBINE, combine_draft_kernel(), dim3(B, gamma), dim3(256), ca);
    if (mem.fixed) return run_direct(c, stream, nodes);
    return run_chain(c, stream, nodes, B, gamma, V, r, (int)wdtype, mode + 16 + (merge_out ? 32 : 0), grid, n_vc);
  }
  const int hs = gru ? 1 : 0;
  const void* kfn = pl.shared ? sweep_kernel((int)wdtype, r, mode, hs ? c->gru_depth : c->draft_depth,
                                             hs ? c->gru_nt : c->draft_nt, hs)
                              : sweep_kernel((int)wdtype, r, mode, 0, 1, hs);
  // Markov: gamma sweeps, each taking x_{k-1} from the previous position's
  // running bests.  GRU: s_0 fill, then per position the sweep (bias from
  // s_{k-1}) and, before the next one, s_k = GRU(s_{k-1}, W1[x_k]).  Then one
  // merge of every position's partials.
  std::vector<KernelNode> nodes;
  nodes.reserve(2 * gamma + 1);
  GruArgs ga;
  if (gru) {
    ga = *gru;
    ga.B = B;
    ga.R = r;
    ga.V = V;
    ga.W1 = W1;
    ga.w1_bf16 = wdtype == DSPARK_BF16;
    ga.states = states;
    ga.err = c->dev_err;
    ga.k = 0;
    KernelNode n;
    set_node(n, DSPARK_K_GRU, gru_init_kernel(), dim3((unsigned)(((int64_t)B * r + 255) / 256)), dim3(256), ga);
    nodes.push_back(n);
    sa.hstate = states;
  }
  for (int k = 1; k <= gamma; ++k) {
    sa.k = k;
    sa.pf = pf + (size_t)(k - 1) * npos;
    sa.pi = pi + (size_t)(k - 1) * npos;
    sa.best = best + (size_t)(k - 1) * kBestGroups * B;
    sa.best_prev = (!gru && k > 1) ? best + (size_t)(k - 2) * kBestGroups * B : nullptr;
    KernelNode n;
    set_node(n, DSPARK_K_DRAFT_SWEEP, kfn, dim3(pl.grid), dim3(256), sa);
    nodes.push_back(n);
    if (gru && k < gamma) {
      ga.k = k;
      ga.best = sa.best;
      set_node(n, DSPARK_K_GRU, gru_step_kernel(r), dim3(r / 16, (B + 15) / 16), dim3(gru_step_threads(r)), ga);
      nodes.push_back(n);
    }
  }
  if (merge_out) {
    *merge_out = ca;
  } else {
    KernelNode n;
    set_node(n, DSPARK_K_DRAFT_COMBINE, combine_draft_kernel(), dim3(B, gamma), dim3(256), ca);
    nodes.push_back(n);
  }
  if (mem.fixed) return run_direct(c, stream, nodes);
  return run_chain(c, stream, nodes, B, gamma, V, r, (int)wdtype, mode + 4 * hs + (merge_out ? 32 : 0), pl.grid,
                   pl.n_vc);
}

int schedule_common(dspark_ctx* c, hipStream_t stream, int B, int gamma, const float* surv, const float* hist,
                    const float* sps, int n_sps, int32_t* K, int32_t* n_selected, double* theta) {
  if (B < 1 || gamma < 1 || gamma > kMaxGamma) return fail(c, DSPARK_EINVAL, "bad shape B=%d gamma=%d", B, gamma);
  if ((long)B * gamma > 4096) return fail(c, DSPARK_EINVAL, "B * gamma must be <= 4096");
  if (n_sps < B) return fail(c, DSPARK_EINVAL, "n_sps (%d) must be >= B (%d)", n_sps, B);
  if (!surv || !sps || !K || !n_selected || !theta) return fail(c, DSPARK_EINVAL, "null pointer argument");
  DeviceGuard dg(c->device);
  if (!dg.ok) return fail(c, DSPARK_EHIP, "hipSetDevice failed");
  SchedArgs a;
  a.B = B;
  a.gamma = gamma;
  a.n_sps = n_sps;
  a.surv = surv;
  a.surv_hist = hist;
  a.sps = sps;
  a.K = K;
  a.n_selected = n_selected;
  a.theta = theta;
  int rc;
  // keys by rank (one or two sets of 4096), then the scan / stop / count
  if ((rc = ensure_ws(c, 2 * 4096 * sizeof(uint64_t)))) return rc;
  a.sorted = static_cast<uint64_t*>(c->ws);
  const int n = B * gamma;
  if ((rc = klaunch(c, DSPARK_K_SCHEDULE, schedule_rank_kernel(), dim3((n + 15) / 16, hist ? 2 : 1),
                    dim3(kSchedThreads), &a, stream)))
    return rc;
  if ((rc = klaunch(c, DSPARK_K_SCHEDULE, schedule_kernel(hist ? 1 : 0), dim3(1), dim3(kSchedThreads), &a, stream)))
    return rc;
  return DSPARK_OK;
}

// Verification of either target layout (toffs null: strided rows; else
// packed rows, request b's rows 1 .. K_b + 1 from row toffs[b] on).
int verify_common(dspark_ctx* c, hipStream_t stream, int B, int gamma, int V, int r, dspark_dtype wdtype,
                  const float* target, int64_t t_stride_b, int64_t t_stride_k, const int32_t* toffs, int t_rows,
                  const float* U,
                  int64_t u_stride_b, int64_t u_stride_k, const void* W1, const void* W2,
                  const int32_t* anchor, const int32_t* tokens, const float* lse, const float* ytok,
                  const float* states, const int32_t* K, const uint32_t* req_ids, float temperature,
                  uint64_t seed, int32_t* accept_len, int32_t* out_tokens) {
  int rc = check_markov_shape(c, B, gamma, V, r, (int)wdtype, temperature);
  if (rc) return rc;
  if (!toffs) {
    if ((rc = check_stream_rows(c, "target", target, t_stride_b, t_stride_k, B, gamma + 1, V))) return rc;
  } else {
    if (!target) return fail(c, DSPARK_EINVAL, "target is NULL");
    if (!aligned16(target)) return fail(c, DSPARK_EINVAL, "target must be 16-byte aligned");
    if (t_stride_k < V || (t_stride_k & 3)) return fail(c, DSPARK_EINVAL, "target row stride must be >= V and a multiple of 4");
  }
  const bool greedy = temperature == 0.0f;
  if (!greedy && (rc = check_stream_rows(c, "U", U, u_stride_b, u_stride_k, B, gamma, V))) return rc;
  if (!tokens || !accept_len || !out_tokens) return fail(c, DSPARK_EINVAL, "null pointer argument");
  if (!greedy && (!W2 || !lse || !ytok || (!states && (!W1 || !anchor))))
    return fail(c, DSPARK_EINVAL, "sampling verification needs U, W2, lse, ytok and W1 + anchor or states");
  if (!greedy && ((W1 && !aligned16(W1)) || !aligned16(W2) || (states && !aligned16(states))))
    return fail(c, DSPARK_EINVAL, "W1, W2 and states must be 16-byte aligned");
  DeviceGuard dg(c->device);
  if (!dg.ok) return fail(c, DSPARK_EHIP, "hipSetDevice failed");

  const int rows = B * (gamma + 1);
  // windows of target rows: the first for every request, each later one only
  // for requests that kept every draft so far
  int win_lo[9], win_hi[9];
  int n_win = 0;
  {
    int lo = 1;
    for (int i = 0; i < 8 && c->verify_win[i] > 0 && c->verify_win[i] < gamma + 1; ++i) {
      win_lo[n_win] = lo;
      win_hi[n_win] = c->verify_win[i];
      lo = c->verify_win[i] + 1;
      ++n_win;
    }
    win_lo[n_win] = lo;
    win_hi[n_win] = gamma + 1;
    ++n_win;
  }
  const int n_chunks = ((V >> 2) + kRowsThreads * kRowsPer - 1) / (kRowsThreads * kRowsPer);
  const SweepPlan pl = plan_sweep(c, B, V, r, (int)wdtype);
  const size_t n_rowpart = (size_t)rows * n_chunks;
  const size_t n_respart = (size_t)B * pl.n_vc;
  size_t off = 0;
  const size_t off_rpf = off;
  off += align256(n_rowpart * sizeof(float4));
  const size_t off_rpi = off;
  off += align256(n_rowpart * sizeof(int));
  const size_t off_spf = off;
  off += align256(n_respart * sizeof(float4));
  const size_t off_spi = off;
  off += align256(n_respart * sizeof(int2));
  const size_t off_rk = off;
  off += align256((size_t)B * sizeof(int32_t));
  const size_t off_rlt = off;
  off += align256((size_t)B * sizeof(float));
  const size_t off_vs = off;
  off += align256((size_t)B * sizeof(int2));
  const size_t off_list = off;                          // two pending-request lists
  off += 2 * align256((size_t)(B + 1) * sizeof(int));
  if ((rc = ensure_ws(c, off))) return rc;
  char* ws = static_cast<char*>(c->ws);
  float4* rpf = reinterpret_cast<float4*>(ws + off_rpf);
  int* rpi = reinterpret_cast<int*>(ws + off_rpi);
  float4* spf = reinterpret_cast<float4*>(ws + off_spf);
  int2* spi = reinterpret_cast<int2*>(ws + off_spi);
  int32_t* resid_k = reinterpret_cast<int32_t*>(ws + off_rk);
  float* resid_lt = reinterpret_cast<float*>(ws + off_rlt);
  int2* vstate = reinterpret_cast<int2*>(ws + off_vs);
  int* lists[2] = {reinterpret_cast<int*>(ws + off_list),
                   reinterpret_cast<int*>(ws + off_list + align256((size_t)(B + 1) * sizeof(int)))};

  const bool vchain = c->verify_chain && c->vchain_wg_per_cu > 0 && n_chunks <= 64;
  const float invT = greedy ? 1.0f : 1.0f / temperature;
  if (vchain) {
    const int np = std::min(kVqMaxPart, B);
    const int per_cu = c->vchain_wg > 0 ? std::min(c->vchain_wg, c->vchain_wg_per_cu) : c->vchain_wg_per_cu;
    const int wp = std::max(1, per_cu * c->cu_count / np);
    const int qcap = ((B + np - 1) / np) * gamma + (wp + n_chunks - 1) / n_chunks + 4;
    if ((rc = ensure_vq(c, vq_words(rows, np, qcap)))) return rc;
    VerifyArgs va;
    memset(&va, 0, sizeof(va));
    va.B = B;
    va.gamma = gamma;
    va.V = V;
    va.n_chunks = n_chunks;
    va.greedy = greedy;
    va.lo = 1;
    va.hi = gamma + 1;
    va.first = 1;                                        // K out of range is reported at row 1
    va.vq = c->vq;
    va.n_part = np;
    va.qcap = qcap;
    va.bar_test = c->bar_test;
    va.lookahead = c->vchain_ahead;
    va.T = target;
    va.tsb = t_stride_b;
    va.toffs = toffs;
    va.t_rows = t_rows;
    va.tsk = t_stride_k;
    va.K = K;
    va.req = req_ids;
    va.tokens = tokens;
    va.lse = lse;
    va.ytok = ytok;
    va.invT = invT;
    va.s2 = greedy ? kLog2e : kLog2e / temperature;
    va.seed = seed;
    va.pf = rpf;
    va.pi = rpi;
    va.accept_len = accept_len;
    va.out_tokens = out_tokens;
    va.resid_k = resid_k;
    va.resid_lt = resid_lt;
    va.err = c->dev_err;
    if ((rc = klaunch(c, DSPARK_K_VERIFY_CHAIN, verify_chain_kernel(), dim3(np * wp), dim3(kRowsThreads), &va,
                      stream)))
      return rc;
    n_win = 0;                                           // no window passes
  }
  for (int w = 0; w < n_win; ++w) {
    const int nrows = win_hi[w] - win_lo[w] + 1;
    VerifyArgs va;
    memset(&va, 0, sizeof(va));
    va.B = B;
    va.gamma = gamma;
    va.V = V;
    va.n_chunks = n_chunks;
    va.greedy = greedy;
    va.lo = win_lo[w];
    va.hi = win_hi[w];
    va.first = w == 0;
    va.vstate = vstate;
    // later windows walk the requests the previous window left pending
    va.list_in = (w > 0 && c->verify_list) ? lists[(w - 1) % 2] : nullptr;
    va.list_out = (w + 1 < n_win && c->verify_list) ? lists[w % 2] : nullptr;
    va.T = target;
    va.tsb = t_stride_b;
    va.toffs = toffs;
    va.t_rows = t_rows;
    va.tsk = t_stride_k;
    va.K = K;
    va.req = req_ids;
    va.tokens = tokens;
    va.lse = lse;
    va.ytok = ytok;
    va.invT = invT;
    va.s2 = greedy ? kLog2e : kLog2e / temperature;
    va.seed = seed;
    va.pf = rpf;
    va.pi = rpi;
    va.accept_len = accept_len;
    va.out_tokens = out_tokens;
    va.resid_k = resid_k;
    va.resid_lt = resid_lt;
    va.err = c->dev_err;
    const long all_tasks = (long)n_chunks * B * nrows;
    const dim3 rgrid = va.list_in ? dim3((unsigned)std::min<long>(all_tasks, 8L * c->cu_count))
                                  : dim3(n_chunks, B * nrows);
    if ((rc = klaunch(c, DSPARK_K_VERIFY_ROWS, verify_rows_kernel(), rgrid, dim3(kRowsThreads), &va, stream)))
      return rc;
    if ((rc = klaunch(c, DSPARK_K_VERIFY_DECIDE, verify_decide_kernel(), dim3(B), dim3(64), &va, stream)))
      return rc;
  }
  if (greedy) return DSPARK_OK;

  SweepArgs sa;
  memset(&sa, 0, sizeof(sa));
  sa.B = B;
  sa.gamma = gamma;
  sa.V = V;
  sa.k = 0;
  sa.n_rg = pl.n_rg;
  sa.n_vc = pl.n_vc;
  sa.n_tiles = pl.n_tiles;
  sa.xcd_remap = 1;
  sa.U = U;
  sa.usb = u_stride_b;
  sa.usk = u_stride_k;
  sa.T = target;
  sa.tsb = t_stride_b;
  sa.toffs = toffs;
  sa.t_rows = t_rows;
  sa.tsk = t_stride_k;
  sa.W1 = W1;
  sa.W2 = W2;
  sa.anchor = anchor;
  sa.tokens = tokens;
  sa.req = req_ids;
  sa.resid_k = resid_k;
  sa.lse = lse;
  sa.resid_lt = resid_lt;
  sa.invT = invT;
  sa.s2 = kLog2e / temperature;
  sa.seed = seed;
  sa.pf = spf;
  sa.pi = spi;
  sa.hstate = states;
  sa.err = c->dev_err;
  const void* rfn = sweep_kernel((int)wdtype, r, kModeResidual, pl.shared ? c->resid_depth : 0,
                                 pl.shared ? c->resid_nt : 1, states ? 1 : 0);
  if ((rc = klaunch(c, DSPARK_K_RESID_SWEEP, rfn, dim3(pl.grid), dim3(256), &sa, stream))) return rc;

  CombineArgs ca;
  memset(&ca, 0, sizeof(ca));
  ca.B = B;
  ca.gamma = gamma;
  ca.V = V;
  ca.n_vc = pl.n_vc;
  ca.pf = spf;
  ca.pi = spi;
  ca.resid_k = resid_k;
  ca.accept_len = accept_len;
  ca.out_tokens = out_tokens;
  ca.err = c->dev_err;
  if ((rc = klaunch(c, DSPARK_K_RESID_COMBINE, combine_resid_kernel(), dim3(B), dim3(256), &ca, stream))) return rc;
  return DSPARK_OK;
}

// Diagnostic pass: per-position acceptance probabilities.
int accept_prob_impl(dspark_ctx* c, hipStream_t stream, int B, int gamma, int V, int r, dspark_dtype wdtype,
                     const float* target, int64_t t_stride_b, int64_t t_stride_k, const float* U,
                     int64_t u_stride_b, int64_t u_stride_k, const void* W1, const void* W2, const int32_t* anchor,
                     const int32_t* tokens, const float* lse, const float* states, float temperature, float* alpha) {
  int rc = check_markov_shape(c, B, gamma, V, r, (int)wdtype, temperature);
  if (rc) return rc;
  if (!(temperature > 0.0f)) return fail(c, DSPARK_EINVAL, "acceptance probabilities need temperature > 0");
  if ((rc = check_stream_rows(c, "target", target, t_stride_b, t_stride_k, B, gamma, V))) return rc;
  if ((rc = check_stream_rows(c, "U", U, u_stride_b, u_stride_k, B, gamma, V))) return rc;
  if (!W2 || !tokens || !lse || !alpha || (!states && (!W1 || !anchor)))
    return fail(c, DSPARK_EINVAL, "null pointer argument");
  if ((W1 && !aligned16(W1)) || !aligned16(W2) || (states && !aligned16(states)))
    return fail(c, DSPARK_EINVAL, "W1, W2 and states must be 16-byte aligned");
  DeviceGuard dg(c->device);
  if (!dg.ok) return fail(c, DSPARK_EHIP, "hipSetDevice failed");

  const int rows = B * (gamma + 1);
  const int n_chunks = ((V >> 2) + kRowsThreads * kRowsPer - 1) / (kRowsThreads * kRowsPer);
  const SweepPlan pl = plan_sweep(c, B, V, r, (int)wdtype);
  const size_t n_rowpart = (size_t)rows * n_chunks;
  const size_t npos = (size_t)B * pl.n_vc;
  size_t off = 0;
  const size_t off_rpf = off;
  off += align256(n_rowpart * sizeof(float4));
  const size_t off_rpi = off;
  off += align256(n_rowpart * sizeof(int));
  const size_t off_lse = off;
  off += align256((size_t)B * gamma * sizeof(float));
  const size_t off_spf = off;
  off += align256(npos * gamma * sizeof(float4));
  if ((rc = ensure_ws(c, off))) return rc;
  char* ws = static_cast<char*>(c->ws);
  float4* rpf = reinterpret_cast<float4*>(ws + off_rpf);
  int* rpi = reinterpret_cast<int*>(ws + off_rpi);
  float* row_lse = reinterpret_cast<float*>(ws + off_lse);
  float4* spf = reinterpret_cast<float4*>(ws + off_spf);

  // 1. log-normaliser of every target row 1..gamma
  VerifyArgs va;
  memset(&va, 0, sizeof(va));
  va.B = B;
  va.gamma = gamma;
  va.V = V;
  va.n_chunks = n_chunks;
  va.lo = 1;
  va.hi = gamma;
  va.first = 1;
  va.T = target;
  va.tsb = t_stride_b;
  va.tsk = t_stride_k;
  va.s2 = kLog2e / temperature;
  va.pf = rpf;
  va.pi = rpi;
  va.row_lse = row_lse;
  va.err = c->dev_err;
  if ((rc = klaunch(c, DSPARK_K_DIAG, verify_rows_kernel(), dim3(n_chunks, B * gamma), dim3(kRowsThreads), &va,
                    stream)))
    return rc;
  if ((rc = klaunch(c, DSPARK_K_DIAG, rows_lse_kernel(), dim3(B, gamma), dim3(64), &va, stream))) return rc;

  // 2. per position, sum over the vocabulary of min(p_t, p_d), the draft row
  //    rebuilt on MFMA as in the draft
  SweepArgs sa;
  memset(&sa, 0, sizeof(sa));
  sa.B = B;
  sa.gamma = gamma;
  sa.V = V;
  sa.n_rg = pl.n_rg;
  sa.n_vc = pl.n_vc;
  sa.n_tiles = pl.n_tiles;
  sa.xcd_remap = 1;
  sa.U = U;
  sa.usb = u_stride_b;
  sa.usk = u_stride_k;
  sa.T = target;
  sa.tsb = t_stride_b;
  sa.tsk = t_stride_k;
  sa.W1 = W1;
  sa.W2 = W2;
  sa.anchor = anchor;
  sa.tokens = tokens;
  sa.lse = lse;
  sa.resid_lt = row_lse;
  sa.hstate = states;
  sa.invT = 1.0f / temperature;
  sa.s2 = kLog2e / temperature;
  sa.err = c->dev_err;
  const void* fn = sweep_kernel((int)wdtype, r, kModeAlpha, pl.shared ? c->resid_depth : 0,
                                pl.shared ? c->resid_nt : 1, states ? 1 : 0);
  for (int k = 1; k <= gamma; ++k) {
    sa.k = k;
    sa.pf = spf + (size_t)(k - 1) * npos;
    if ((rc = klaunch(c, DSPARK_K_DIAG, fn, dim3(pl.grid), dim3(256), &sa, stream))) return rc;
  }
  CombineArgs ca;
  memset(&ca, 0, sizeof(ca));
  ca.B = B;
  ca.gamma = gamma;
  ca.V = V;
  ca.n_vc = pl.n_vc;
  ca.pf = spf;
  ca.lse = alpha;
  ca.err = c->dev_err;
  return klaunch(c, DSPARK_K_DIAG, combine_alpha_kernel(), dim3(B, gamma), dim3(256), &ca, stream);
}

// Host trace ranges (roctx) around the entry points, for a profiler's marker
// trace (rocprofv3 --marker-trace): on when DSPARK_ROCTX=1 is set as the
// library first makes a call, resolved at run time (no link dependency).
// Off, a range costs one test of a cached pointer.
namespace {
typedef int (*roctx_push_fn)(const char*);
typedef int (*roctx_pop_fn)();
struct RoctxApi {
  roctx_push_fn push = nullptr;
  roctx_pop_fn pop = nullptr;
};

RoctxApi roctx_load() {
  RoctxApi a;
  const char* e = getenv("DSPARK_ROCTX");
  if (!e || e[0] != '1') return a;
  void* h = dlopen("librocprofiler-sdk-roctx.so.1", RTLD_NOW | RTLD_LOCAL);
  if (!h) h = dlopen("librocprofiler-sdk-roctx.so", RTLD_NOW | RTLD_LOCAL);
  if (!h) return a;
  a.push = reinterpret_cast<roctx_push_fn>(dlsym(h, "roctxRangePushA"));
  a.pop = reinterpret_cast<roctx_pop_fn>(dlsym(h, "roctxRangePop"));
  if (!a.push || !a.pop) a = RoctxApi();
  return a;
}

const RoctxApi& roctx() {
  static const RoctxApi a = roctx_load();
  return a;
}

struct TraceRange {
  bool on;
  explicit TraceRange(const char* name) : on(roctx().push != nullptr) {
    if (on) roctx().push(name);
  }
  ~TraceRange() {
    if (on) roctx().pop();
  }
};
}  // namespace

extern "C" {

int dspark_version(void) { return kVersion; }

int dspark_create(dspark_ctx** out, int device) {
  if (!out) return DSPARK_EINVAL;
  *out = nullptr;
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || device < 0 || device >= n) {
    (void)hipGetLastError();
    return DSPARK_EHIP;
  }
  DeviceGuard dg(device);
  if (!dg.ok) return DSPARK_EHIP;
  dspark_ctx* c = new dspark_ctx();
  c->device = device;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, device) == hipSuccess && prop.multiProcessorCount > 0)
    c->cu_count = prop.multiProcessorCount;
  if (hipMalloc(&c->dev_err, 1024) != hipSuccess || hipMemset(c->dev_err, 0, 1024) != hipSuccess) {
    (void)hipGetLastError();
    delete c;
    return DSPARK_EHIP;
  }
  c->bar = reinterpret_cast<unsigned int*>(reinterpret_cast<char*>(c->dev_err) + 128);
  c->chain = reinterpret_cast<unsigned int*>(reinterpret_cast<char*>(c->dev_err) + 512);
  if (hipMalloc(&c->chain_flags, (size_t)kChainMaxGrid * 128) != hipSuccess ||
      hipMemset(c->chain_flags, 0, (size_t)kChainMaxGrid * 128) != hipSuccess) {
    (void)hipGetLastError();
    (void)hipFree(c->dev_err);
    if (c->chain_flags) (void)hipFree(c->chain_flags);
    delete c;
    return DSPARK_EHIP;
  }
  scratch_setup(device);
  // chained draft kernel (every position in one launch, 65..128 requests):
  // "0" switches it off (per-position sweeps)
  const char* ch = getenv("DSPARK_CHAIN");
  if (ch && ch[0] == '0' && ch[1] == 0) c->use_chain = false;
  // its shape: "<waves>,<rows per wave>,<depth>,<chunks>" (e.g. 8,16,3,256)
  const char* cs = getenv("DSPARK_CHAIN_SHAPE");
  if (cs) {
    int wv = 0, rw = 0, dp = 0, ck = 0;
    if (sscanf(cs, "%d,%d,%d,%d", &wv, &rw, &dp, &ck) == 4 && draft_chain_kernel(256, kModeDraftSample, dp, 2, rw, wv) &&
        ck >= 0 && ck <= 4096) {
      c->chain_waves = wv;
      c->chain_rows = rw;
      c->chain_depth = dp;
      c->chain_chunks = ck;
    }
  }
  // whole-draft kernel: "0" never, "1" small batches (default), "2" every
  // eligible batch (up to 128 requests)
  const char* pk = getenv("DSPARK_PERSIST");
  if (pk && pk[0] == '0' && pk[1] == 0) c->persist_max_b = 0;
  if (pk && pk[0] == '2' && pk[1] == 0) c->persist_max_b = 128;
  // whole-draft kernel: "0" launches it plainly instead of cooperatively
  const char* pc = getenv("DSPARK_PERSIST_COOP");
  if (pc && pc[0] == '0' && pc[1] == 0) c->persist_coop = false;
  // failure injection for tests: every grid barrier of the whole-draft kernel
  // and every wait of the chained draft waits for a release that never comes
  // and gives up after 64 polls (the kernels still end; the call's results
  // are invalid and the error flag is raised)
  const char* bt = getenv("DSPARK_BARRIER_TEST");
  if (bt && bt[0] == '1' && bt[1] == 0) c->bar_test = 1;
  // The draft loop goes kernel by kernel by default: on this runtime a
  // stream operation after a graph launch starts ~9 us after the graph's
  // last kernel, more than the graph saves on eight launches of 8-30 us.
  // DSPARK_GRAPH=1 runs it through a cached graph instead.
  const char* g = getenv("DSPARK_GRAPH");
  if (g && g[0] == '1') c->use_graph = true;
  // tuning knob: target resident waves per CU for the vocabulary sweeps
  const char* w = getenv("DSPARK_SWEEP_WAVES_PER_CU");
  if (w) {
    const int v = atoi(w);
    if (v >= 1 && v <= 32) c->sweep_waves_per_cu = v;
  }
  // tuning knobs of the shared-tile sweeps: "<nt>,<depth>" (nt 1 with depth
  // 1..3, or nt 2 with depth 1..2)
  auto ring_knob = [](const char* name, int& nt, int& depth) {
    const char* v = getenv(name);
    if (!v || v[0] < '1' || v[0] > '2' || v[1] != ',' || v[2] < '1' || v[2] > '3' || v[3] != 0) return;
    if (v[0] == '2' && v[2] == '3') return;
    nt = v[0] - '0';
    depth = v[2] - '0';
  };
  ring_knob("DSPARK_DRAFT_RING", c->draft_nt, c->draft_depth);
  ring_knob("DSPARK_GRU_RING", c->gru_nt, c->gru_depth);
  ring_knob("DSPARK_RESID_RING", c->resid_nt, c->resid_depth);
  // verify windows: "e1,e2,..." increasing last rows of all windows but the final one
  const char* sw = getenv("DSPARK_STS_WG_PER_CU");
  if (sw) {
    const int v = atoi(sw);
    if (v >= 1 && v <= 16) c->sts_wg_per_cu = v;
  }
  const char* vl = getenv("DSPARK_VERIFY_LIST");
  if (vl && vl[0] == '0' && vl[1] == 0) c->verify_list = false;
  const char* vc = getenv("DSPARK_VERIFY_CHAIN");
  if (vc && vc[1] == 0 && (vc[0] == '0' || vc[0] == '1')) c->verify_chain = vc[0] == '1';
  const char* vca = getenv("DSPARK_VERIFY_AHEAD");
  if (vca) {
    const int v = atoi(vca);
    if (v >= 1 && v <= 8) c->vchain_ahead = v;
  }
  const char* vcw = getenv("DSPARK_VERIFY_CHAIN_WG");
  if (vcw) {
    const int v = atoi(vcw);
    if (v >= 1 && v <= 16) c->vchain_wg = v;
  }
  const char* vw = getenv("DSPARK_VERIFY_WINDOWS");
  if (vw) {
    int tmp[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    int n = 0, prev = 0;
    bool ok = true;
    for (const char* q = vw; *q && ok;) {
      char* end = nullptr;
      const long v = strtol(q, &end, 10);
      if (end == q || v <= prev || v > 64 || n >= 7) ok = false;
      else {
        tmp[n++] = (int)v;
        prev = (int)v;
        q = (*end == ',') ? end + 1 : end;
        if (*end && *end != ',') ok = false;
      }
    }
    if (ok) memcpy(c->verify_win, tmp, sizeof(tmp));
  }
  // resident workgroups per CU of the chained draft (its grid), asked once
  {
    int nb = 0;
    const void* fn = draft_chain_kernel(256, kModeDraftSample, c->chain_depth, 2, c->chain_rows, c->chain_waves);
    if (fn && hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fn, 64 * c->chain_waves, 0) != hipSuccess) {
      (void)hipGetLastError();
      nb = 0;
    }
    c->chain_wg_per_cu = nb;
  }
  // resident workgroups per CU of the verify chain (its grid)
  {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, verify_chain_kernel(), kRowsThreads, 0) != hipSuccess) {
      (void)hipGetLastError();
      nb = 0;
    }
    c->vchain_wg_per_cu = nb;
  }
  *out = c;
  return DSPARK_OK;
}

void dspark_destroy(dspark_ctx* c) {
  if (!c) return;
  {
    DeviceGuard dg(c->device);
    (void)hipDeviceSynchronize();
    for (auto& g : c->graphs) {
      if (g.exec) (void)hipGraphExecDestroy(g.exec);
      if (g.graph) (void)hipGraphDestroy(g.graph);
    }
    for (auto& p : c->pending) {
      (void)hipEventDestroy(p.a);
      (void)hipEventDestroy(p.b);
    }
    for (auto e : c->ev_free) (void)hipEventDestroy(e);
    if (c->ws) (void)hipFree(c->ws);
    if (c->best) (void)hipFree(c->best);
    if (c->sts_buf) (void)hipFree(c->sts_buf);
    if (c->dev_err) (void)hipFree(c->dev_err);
    if (c->chain_flags) (void)hipFree(c->chain_flags);
    if (c->vq) (void)hipFree(c->vq);
    if (c->cm_cnt) (void)hipFree(c->cm_cnt);
  }
  delete c;
}

const char* dspark_last_error(const dspark_ctx* c) { return c ? c->err.c_str() : "null context"; }

int dspark_check(dspark_ctx* c, hipStream_t stream) {
  TraceRange trace_range("dspark_check");
  if (!c) return DSPARK_EINVAL;
  DeviceGuard dg(c->device);
  if (!dg.ok) return fail(c, DSPARK_EHIP, "hipSetDevice failed");
  DSPARK_HIP(c, hipStreamSynchronize(stream));
  int32_t flag = 0;
  DSPARK_HIP(c, hipMemcpy(&flag, c->dev_err, sizeof(flag), hipMemcpyDeviceToHost));
  if (flag) {
    DSPARK_HIP(c, hipMemset(c->dev_err, 0, sizeof(int32_t)));
    return fail(c, DSPARK_EDEVICE, "device error flag 0x%x:%s%s%s%s%s%s", flag,
                (flag & kErrToken) ? " token id out of range" : "",
                (flag & kErrK) ? " verify length out of range" : "",
                (flag & kErrRow) ? " packed target row out of range" : "",
                (flag & kErrBarrier) ? " grid barrier timed out" : "",
                (flag & kErrGrid) ? " candidate temperature not positive and finite" : "",
                (flag & kErrLen) ? " accepted length out of range" : "");
  }
  c->err.clear();
  return DSPARK_OK;
}

int dspark_timing_enable(dspark_ctx* c, int enable) {
  if (!c) return DSPARK_EINVAL;
  c->timing = enable != 0;
  return DSPARK_OK;
}

int dspark_timing_read(dspark_ctx* c, double* ms, int* launches) {
  if (!c || !ms || !launches) return DSPARK_EINVAL;
  DeviceGuard dg(c->device);
  if (!dg.ok) return fail(c, DSPARK_EHIP, "hipSetDevice failed");
  for (int i = 0; i < DSPARK_K_COUNT; ++i) {
    ms[i] = 0.0;
    launches[i] = 0;
  }
  int rc = DSPARK_OK;
  for (auto& p : c->pending) {
    float t = 0.f;
    if (rc == DSPARK_OK) {
      hipError_t e = hipEventSynchronize(p.b);
      if (e == hipSuccess) e = hipEventElapsedTime(&t, p.a, p.b);
      if (e != hipSuccess) rc = fail(c, DSPARK_EHIP, "event timing failed: %s", hipGetErrorString(e));
    }
    if (p.cls >= 0 && p.cls < DSPARK_K_COUNT) {
      ms[p.cls] += t;
      launches[p.cls] += 1;
    }
    c->ev_free.push_back(p.a);
    c->ev_free.push_back(p.b);
  }
  c->pending.clear();
  return rc;
}

int dspark_draft_markov(dspark_ctx* c, hipStream_t stream, int B, int gamma, int V, int r,
                        dspark_dtype wdtype, const float* U, int64_t u_stride_b, int64_t u_stride_k,
                        const void* W1, const void* W2, const int32_t* anchor, const uint32_t* req_ids,
                        float temperature, uint64_t seed, int32_t* tokens, float* lse, float* ytok) {
  TraceRange trace_range("dspark_draft_markov");
  if (!c) return DSPARK_EINVAL;
  if (!anchor) return fail(c, DSPARK_EINVAL, "null pointer argument");
  return draft_chain(c, stream, B, gamma, V, r, wdtype, U, u_stride_b, u_stride_k, W1, W2, anchor, nullptr,
                     req_ids, temperature, seed, tokens, lse, ytok, nullptr);
}

int dspark_draft_markov_static(dspark_ctx* c, hipStream_t stream, int B, int gamma, int V, int r,
                               dspark_dtype wdtype, const float* U, int64_t u_stride_b, int64_t u_stride_k,
                               const void* W1, const void* W2, const int32_t* anchor, const uint32_t* req_ids,
                               float temperature, uint64_t seed, int32_t* tokens, float* lse, float* ytok) {
  TraceRange trace_range("dspark_draft_markov_static");
  if (!c) return DSPARK_EINVAL;
  if (!anchor) return fail(c, DSPARK_EINVAL, "null pointer argument");
  DraftMem mem;
  mem.fixed = true;
  mem.base = static_cast<unsigned char*>(scratch_ptr(c->device));
  if (!mem.base) return fail(c, DSPARK_EHIP, "the static scratch of device %d has no device address", c->device);
  return draft_chain(c, stream, B, gamma, V, r, wdtype, U, u_stride_b, u_stride_k, W1, W2, anchor, nullptr,
                     req_ids, temperature, seed, tokens, lse, ytok, nullptr, mem);
}

int dspark_draft_rnn(dspark_ctx* c, hipStream_t stream, int B, int gamma, int V, int r, dspark_dtype wdtype,
                     const float* U, int64_t u_stride_b, int64_t u_stride_k, const void* W1, const void* W2,
                     const void* W_ih, const void* W_hh, const void* b_ih, const void* b_hh, const void* s0,
                     const uint32_t* req_ids, float temperature, uint64_t seed, int32_t* tokens, float* lse,
                     float* ytok, float* states) {
  TraceRange trace_range("dspark_draft_rnn");
  if (!c) return DSPARK_EINVAL;
  if (!W_ih || !W_hh || !b_ih || !b_hh || !s0 || !states)
    return fail(c, DSPARK_EINVAL, "null pointer argument");
  if (!aligned16(W_ih) || !aligned16(W_hh) || !aligned16(states))
    return fail(c, DSPARK_EINVAL, "W_ih, W_hh and states must be 16-byte aligned");
  GruArgs g;
  memset(&g, 0, sizeof(g));
  g.W_ih = static_cast<const uint16_t*>(W_ih);
  g.W_hh = static_cast<const uint16_t*>(W_hh);
  g.b_ih = static_cast<const uint16_t*>(b_ih);
  g.b_hh = static_cast<const uint16_t*>(b_hh);
  g.s0 = static_cast<const uint16_t*>(s0);
  return draft_chain(c, stream, B, gamma, V, r, wdtype, U, u_stride_b, u_stride_k, W1, W2, nullptr, &g,
                     req_ids, temperature, seed, tokens, lse, ytok, states);
}

namespace {

int check_confidence(dspark_ctx* c, int B, int gamma, int V, int d_h, int d_e, const void* h, const void* E,
                     const int32_t* anchor, const int32_t* tokens, const void* wc, float bc, float* conf,
                     float* surv) {
  if (B < 1 || gamma < 1 || gamma > kMaxGamma || V < 1)
    return fail(c, DSPARK_EINVAL, "bad shape B=%d gamma=%d V=%d", B, gamma, V);
  if (d_h < 8 || d_e < 8 || (d_h & 7) || (d_e & 7))
    return fail(c, DSPARK_EINVAL, "d_h and d_e must be positive multiples of 8");
  if (!h || !E || !anchor || !tokens || !wc || !conf || !surv)
    return fail(c, DSPARK_EINVAL, "null pointer argument");
  if (!aligned16(h) || !aligned16(E) || !aligned16(wc))
    return fail(c, DSPARK_EINVAL, "h, E and wc must be 16-byte aligned");
  if (!std::isfinite(bc)) return fail(c, DSPARK_EINVAL, "bc must be finite");
  return DSPARK_OK;
}

ConfArgs conf_args(dspark_ctx* c, int B, int gamma, int V, int d_h, int d_e, const void* h, const void* E,
                   const int32_t* anchor, const int32_t* tokens, const void* wc, float bc, const float* sts_T,
                   float* conf, float* surv) {
  ConfArgs a;
  memset(&a, 0, sizeof(a));
  a.B = B;
  a.gamma = gamma;
  a.V = V;
  a.dh = d_h;
  a.de = d_e;
  a.h = static_cast<const uint16_t*>(h);
  a.E = static_cast<const uint16_t*>(E);
  a.anchor = anchor;
  a.tokens = tokens;
  a.wc = static_cast<const uint16_t*>(wc);
  a.bc = bc;
  a.sts = sts_T;
  a.conf = conf;
  a.surv = surv;
  a.err = c->dev_err;
  return a;
}

}  // namespace

int dspark_confidence(dspark_ctx* c, hipStream_t stream, int B, int gamma, int V, int d_h, int d_e,
                      const void* h, const void* E, const int32_t* anchor, const int32_t* tokens,
                      const void* wc, float bc, const float* sts_T, float* conf, float* surv) {
  TraceRange trace_range("dspark_confidence");
  if (!c) return DSPARK_EINVAL;
  int rc = check_confidence(c, B, gamma, V, d_h, d_e, h, E, anchor, tokens, wc, bc, conf, surv);
  if (rc) return rc;
  DeviceGuard dg(c->device);
  if (!dg.ok) return fail(c, DSPARK_EHIP, "hipSetDevice failed");
  ConfArgs a = conf_args(c, B, gamma, V, d_h, d_e, h, E, anchor, tokens, wc, bc, sts_T, conf, surv);
  // confidences and survival products in one launch, a workgroup per request
  return klaunch(c, DSPARK_K_CONFIDENCE, confidence_kernel(), dim3(B), dim3(1024), &a, stream);
}

int dspark_draft_markov_conf(dspark_ctx* c, hipStream_t stream, int B, int gamma, int V, int r,
                             dspark_dtype wdtype, const float* U, int64_t u_stride_b, int64_t u_stride_k,
                             const void* W1, const void* W2, const int32_t* anchor, const uint32_t* req_ids,
                             float temperature, uint64_t seed, int d_h, int d_e, const void* h, const void* E,
                             const void* wc, float bc, const float* sts_T, int32_t* tokens, float* lse,
                             float* ytok, float* conf, float* surv) {
  TraceRange trace_range("dspark_draft_markov_conf");
  if (!c) return DSPARK_EINVAL;
  int rc = check_confidence(c, B, gamma, V, d_h, d_e, h, E, anchor, tokens, wc, bc, conf, surv);
  if (rc) return rc;
  {
    // the counters first: once the draft is enqueued without its combine,
    // the merge launch below is what leaves the draft's counters at zero
    DeviceGuard dg(c->device);
    if (!dg.ok) return fail(c, DSPARK_EHIP, "hipSetDevice failed");
    if ((rc = ensure_cm(c, (size_t)B))) return rc;
  }
  CombineArgs m;
  memset(&m, 0, sizeof(m));
  if ((rc = draft_chain(c, stream, B, gamma, V, r, wdtype, U, u_stride_b, u_stride_k, W1, W2, anchor, nullptr,
                        req_ids, temperature, seed, tokens, lse, ytok, nullptr, DraftMem(), &m)))
    return rc;
  DeviceGuard dg(c->device);
  if (!dg.ok) return fail(c, DSPARK_EHIP, "hipSetDevice failed");
  ConfMergeArgs a;
  a.m = m;
  a.f = conf_args(c, B, gamma, V, d_h, d_e, h, E, anchor, tokens, wc, bc, sts_T, conf, surv);
  a.cnt = c->cm_cnt;
  // the draft's merge and the confidences, a workgroup per (request, position)
  return klaunch(c, DSPARK_K_CONF_MERGE, conf_merge_kernel(), dim3(B, gamma), dim3(384), &a, stream);
}

int dspark_schedule(dspark_ctx* c, hipStream_t stream, int B, int gamma, const float* surv,
                    const float* sps, int n_sps, int32_t* K, int32_t* n_selected, double* theta) {
  TraceRange trace_range("dspark_schedule");
  if (!c) return DSPARK_EINVAL;
  return schedule_common(c, stream, B, gamma, surv, nullptr, sps, n_sps, K, n_selected, theta);
}

int dspark_schedule_async(dspark_ctx* c, hipStream_t stream, int B, int gamma, const float* surv,
                          const float* surv_hist, const float* sps, int n_sps, int32_t* K, int32_t* n_selected,
                          double* theta) {
  TraceRange trace_range("dspark_schedule_async");
  if (!c) return DSPARK_EINVAL;
  if (!surv_hist) return fail(c, DSPARK_EINVAL, "null pointer argument");
  return schedule_common(c, stream, B, gamma, surv, surv_hist, sps, n_sps, K, n_selected, theta);
}

int dspark_verify(dspark_ctx* c, hipStream_t stream, int B, int gamma, int V, int r, dspark_dtype wdtype,
                  const float* target, int64_t t_stride_b, int64_t t_stride_k, const float* U,
                  int64_t u_stride_b, int64_t u_stride_k, const void* W1, const void* W2,
                  const int32_t* anchor, const int32_t* tokens, const float* lse, const float* ytok,
                  const float* states, const int32_t* K, const uint32_t* req_ids, float temperature,
                  uint64_t seed, int32_t* accept_len, int32_t* out_tokens) {
  TraceRange trace_range("dspark_verify");
  if (!c) return DSPARK_EINVAL;
  return verify_common(c, stream, B, gamma, V, r, wdtype, target, t_stride_b, t_stride_k, nullptr, 0, U, u_stride_b,
                       u_stride_k, W1, W2, anchor, tokens, lse, ytok, states, K, req_ids, temperature, seed,
                       accept_len, out_tokens);
}

int dspark_accept_prob(dspark_ctx* c, hipStream_t stream, int B, int gamma, int V, int r, dspark_dtype wdtype,
                       const float* target, int64_t t_stride_b, int64_t t_stride_k, const float* U,
                       int64_t u_stride_b, int64_t u_stride_k, const void* W1, const void* W2,
                       const int32_t* anchor, const int32_t* tokens, const float* lse, const float* states,
                       float temperature, float* alpha) {
  TraceRange trace_range("dspark_accept_prob");
  if (!c) return DSPARK_EINVAL;
  return accept_prob_impl(c, stream, B, gamma, V, r, wdtype, target, t_stride_b, t_stride_k, U, u_stride_b,
                          u_stride_k, W1, W2, anchor, tokens, lse, states, temperature, alpha);
}

int dspark_verify_packed(dspark_ctx* c, hipStream_t stream, int B, int gamma, int V, int r, dspark_dtype wdtype,
                         const float* target, int64_t t_row_stride, const int32_t* t_offsets, int n_rows,
                         const float* U, int64_t u_stride_b, int64_t u_stride_k, const void* W1, const void* W2,
                         const int32_t* anchor, const int32_t* tokens, const float* lse, const float* ytok,
                         const float* states, const int32_t* K, const uint32_t* req_ids, float temperature,
                         uint64_t seed, int32_t* accept_len, int32_t* out_tokens) {
  TraceRange trace_range("dspark_verify_packed");
  if (!c) return DSPARK_EINVAL;
  if (!t_offsets || !K) return fail(c, DSPARK_EINVAL, "the packed layout needs t_offsets and K");
  if (n_rows < 1) return fail(c, DSPARK_EINVAL, "n_rows must be >= 1");
  return verify_common(c, stream, B, gamma, V, r, wdtype, target, 0, t_row_stride, t_offsets, n_rows, U, u_stride_b,
                       u_stride_k, W1, W2, anchor, tokens, lse, ytok, states, K, req_ids, temperature, seed,
                       accept_len, out_tokens);
}

int dspark_sts_fit(dspark_ctx* c, hipStream_t stream, int64_t N, int gamma, const float* logit, int64_t stride,
                   const int32_t* accept_len, const float* grid, int n_grid, int n_bins, float* T, int32_t* index,
                   double* ece) {
  TraceRange trace_range("dspark_sts_fit");
  if (!c) return DSPARK_EINVAL;
  if (N < 0 || gamma < 1 || gamma > kMaxGamma)
    return fail(c, DSPARK_EINVAL, "bad shape N=%lld gamma=%d", (long long)N, gamma);
  if (stride < gamma) return fail(c, DSPARK_EINVAL, "stride must be >= gamma");
  if (n_grid < 1 || n_grid > kStsMaxGrid || n_bins < 1 || n_bins > kStsMaxBins || n_grid * n_bins > kStsMaxCells)
    return fail(c, DSPARK_EINVAL, "need 1 <= n_grid <= %d, 1 <= n_bins <= %d, n_grid * n_bins <= %d", kStsMaxGrid,
                kStsMaxBins, kStsMaxCells);
  if (!grid || !T || !index || !ece || (N > 0 && (!logit || !accept_len)))
    return fail(c, DSPARK_EINVAL, "null pointer argument");
  if (N >= (int64_t)1 << 33) return fail(c, DSPARK_EINVAL, "N must be < 2^33");
  DeviceGuard dg(c->device);
  if (!dg.ok) return fail(c, DSPARK_EHIP, "hipSetDevice failed");
  int rc;
  const int cells = n_grid * n_bins;
  if (!c->sts_buf) {
    const size_t bytes = (kStsMaxCells + 32) * sizeof(unsigned long long);
    if (hipMalloc(&c->sts_buf, bytes) != hipSuccess) {
      (void)hipGetLastError();
      c->sts_buf = nullptr;
      return fail(c, DSPARK_ENOMEM, "allocation of %zu bytes failed", bytes);
    }
    DSPARK_HIP(c, hipMemset(c->sts_buf, 0, bytes));
    DSPARK_HIP(c, hipDeviceSynchronize());
  }
  StsArgs a;
  memset(&a, 0, sizeof(a));
  a.N = N;
  a.gamma = gamma;
  a.n_grid = n_grid;
  a.n_bins = n_bins;
  a.stride = stride;
  a.logit = logit;
  a.len = accept_len;
  a.grid = grid;
  a.T = T;
  a.index = index;
  a.ece = ece;
  a.hist = c->sts_buf;
  a.done = reinterpret_cast<unsigned int*>(c->sts_buf + kStsMaxCells);
  a.err = c->dev_err;
  const int64_t blocks = (N + kStsWaves * 64 - 1) / (kStsWaves * 64);
  const int nwg = (int)std::max<int64_t>(1, std::min<int64_t>(blocks, (int64_t)c->sts_wg_per_cu * c->cu_count));
  for (int k = 1; k <= gamma; ++k) {
    a.k = k;
    if ((rc = klaunch(c, DSPARK_K_STS, sts_hist_kernel((n_grid + 63) / 64, cells), dim3(nwg), dim3(kStsThreads), &a,
                      stream)))
      return rc;
  }
  return DSPARK_OK;
}

int dspark_stream_read(dspark_ctx* c, hipStream_t stream, const float* x, int64_t n, float* out) {
  TraceRange trace_range("dspark_stream_read");
  if (!c) return DSPARK_EINVAL;
  if (n < 0) return fail(c, DSPARK_EINVAL, "n must be >= 0");
  if (!out || (n > 0 && !x)) return fail(c, DSPARK_EINVAL, "null pointer argument");
  if (x && !aligned16(x)) return fail(c, DSPARK_EINVAL, "x must be 16-byte aligned");
  DeviceGuard dg(c->device);
  if (!dg.ok) return fail(c, DSPARK_EHIP, "hipSetDevice failed");
  // sixteen workgroups per CU, fewer when there are not that many float4s
  const int64_t n4 = n / 4;
  const int64_t want = (n4 + kStreamThreads - 1) / kStreamThreads;
  const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(16L * c->cu_count, want));
  int rc;
  if ((rc = ensure_ws(c, (size_t)grid * sizeof(float)))) return rc;
  StreamArgs a;
  memset(&a, 0, sizeof(a));
  a.x = x;
  a.n = n;
  a.n4 = n4;
  a.partials = static_cast<float*>(c->ws);
  a.n_part = grid;
  a.out = out;
  if ((rc = klaunch(c, DSPARK_K_DIAG, stream_read_kernel(), dim3(grid), dim3(kStreamThreads), &a, stream))) return rc;
  return klaunch(c, DSPARK_K_DIAG, stream_sum_kernel(), dim3(1), dim3(kStreamThreads), &a, stream);
}

}  // extern "C"
