// Kernel argument blocks and kernel lookup shared by the translation units of
// libdspark.  Every kernel takes one argument block by value, so a launch (or
// a HIP graph kernel node) is described by (function, grid, block, &args).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dspark {

// Work decomposition of the vocabulary sweeps that carry the Markov bias:
// waves own 32 request rows (two 16-row MFMA blocks) and a contiguous range
// of 16-wide vocabulary tiles; four waves per 256-thread workgroup.
constexpr int kRowsPerWave = 32;
constexpr int kTileV = 16;
constexpr int kWavesPerBlock = 4;
constexpr int kBestGroups = 16;

// kModeAlpha: the acceptance probability sum_v min(p_t, p_d) of every
// request at one position (a diagnostic pass; resid_lt then holds the
// target log-normalisers [B][gamma]).
enum SweepMode : int { kModeDraftGreedy = 0, kModeDraftSample = 1, kModeResidual = 2, kModeAlpha = 3 };

struct SweepArgs {
  int B, gamma, V, k;            // k: 1-based draft position (draft modes)
  int n_rg, n_vc, n_tiles;       // row groups, vocabulary chunks, 16-wide tiles
  int xcd_remap;                 // map blocks sharing a chunk onto one XCD
  const float* U;
  int64_t usb, usk;
  const float* T;                // target logits (residual mode)
  int64_t tsb, tsk;
  const int32_t* toffs;          // packed target rows: first row of each request, or null
  int t_rows;                    // rows of the packed target
  const void* W1;
  const void* W2;
  const int32_t* anchor;
  const int32_t* tokens;         // [B][gamma]
  const uint32_t* req;           // nullable
  const int32_t* resid_k;        // residual mode: 1-based position or 0
  const float* lse;              // residual mode: draft log-normalisers [B][gamma]
  const float* resid_lt;         // residual mode: target log-normaliser per request
  float invT, s2;                // 1/T and log2(e)/T (greedy: 1 and log2 e)
  uint64_t seed;
  float4* pf;                    // partials [B][n_vc]
  int2* pi;
  // draft modes: running best (key, index) of each request at this position,
  // packed so that a larger integer is the winner (see pack_best), kept in
  // kBestGroups slot groups [kBestGroups][B] (chunk vc updates group
  // vc % kBestGroups, which spreads the atomics); and the same for the
  // previous position (its token feeds this one), null at k = 1
  unsigned long long* best;
  const unsigned long long* best_prev;
  // GRU head: fp32 states [gamma][B][r]; position k projects hstate[k-1][b]
  // instead of W1[x_{k-1}] (kernels built with the state bias source)
  const float* hstate;
  // whole-draft kernel: grid barrier arrival counter (zero at launch), and a
  // failure-injection switch for tests (nonzero: every barrier waits for one
  // arrival too many and gives up after 64 polls)
  unsigned int* bar;
  int bar_test;
  // chained draft: [0] ticket counter, [32 + k] finished items of position
  // k (zero at launch; the draft combine clears them); per-workgroup release
  // flags (word 32 b of workgroup b: the last position released, zero at
  // launch and cleared again by the launch's last item)
  unsigned int* chain;
  unsigned int* chain_flags;
  int32_t* err;
};

struct CombineArgs {
  int B, gamma, V, k, n_vc, greedy;
  float invT;
  const float4* pf;              // draft: [gamma][B][n_vc] (every position at once)
  const int2* pi;
  unsigned long long* best;      // draft: [gamma][kBestGroups][B] running bests, cleared here
  unsigned int* bar;             // draft: the whole-draft kernel's barrier counter, reset here (nullable)
  unsigned int* chain;           // draft: the chained kernel's counters, reset here (nullable)
  int32_t* tokens;               // draft: [B][gamma]
  float* lse;
  float* ytok;
  // residual combine
  const int32_t* resid_k;
  const int32_t* accept_len;
  int32_t* out_tokens;           // [B][gamma+1]
  int32_t* err;
};

// Verify row pass of one window (rows lo .. hi, 1-based).
constexpr int kRowsThreads = 256;
constexpr int kRowsPer = 8;      // float4 per thread per chunk: chunks of 2048 float4 (32 KB)

struct VerifyArgs {
  int B, gamma, V, n_chunks, greedy;
  int lo, hi;                    // 1-based rows of this window
  int first;                     // first window: every request starts at row 1
  int2* vstate;                  // per request {accepted so far, next row (0 = done)}
  // later windows: the requests still pending ([0] = count, then their ids),
  // appended by the previous window's decisions; null = one workgroup per
  // (chunk, request, row) of the window.  list_out: where this window's
  // decisions append (its count is cleared by this window's rows pass), or
  // null for the last window.
  const int* list_in;
  int* list_out;
  const float* T;
  int64_t tsb, tsk;
  const int32_t* toffs;          // packed target rows: first row of each request, or null
  int t_rows;                    // rows of the packed target
  const int32_t* K;
  const uint32_t* req;
  const int32_t* tokens;
  const float* lse;
  const float* ytok;
  float invT, s2;                // 1/T and log2(e)/T (greedy: 1 and log2 e)
  uint64_t seed;
  float4* pf;                    // [B*(gamma+1)][n_chunks]: m2, s, key, (verify chain) t at the token
  int* pi;
  int32_t* accept_len;
  int32_t* out_tokens;
  int32_t* resid_k;
  float* resid_lt;
  float* row_lse;                // diagnostic pass: ln sum exp(t/T) of rows 1..gamma, [B][gamma]
  // verify chain (every row in one launch): its counter block (layout in
  // verify.hip, zero at launch and left zero), the request partitions and
  // the row slots per partition; bar_test: every wait for a row gives up
  // after 64 polls (failure injection from the host)
  unsigned int* vq;
  int n_part, qcap, bar_test;
  int lookahead;                 // rows of a request in flight ahead of its decisions (>= 1)
  int32_t* err;
};
// Counter block of the verify chain, in 32-bit words: per partition p a
// ticket counter, a row-queue tail, a count of decided requests and the last
// row slot any ticket may wait on, each on its own 128-byte line; an exit
// counter and an abort flag; one finished-chunk counter per target row
// (64-byte stride); then the row slots of each partition, one 128-byte line
// each (a slot is polled by the workgroups holding its tickets).
constexpr int kVqPartWords = 128;
constexpr int kVqMaxPart = 8;
constexpr int kVqExit = kVqMaxPart * kVqPartWords;
constexpr int kVqAbort = kVqExit + 32;
constexpr int kVqRows = kVqExit + 128;
constexpr int kVqRowStride = 16;
constexpr int kVqSlotStride = 32;
__host__ __device__ constexpr size_t vq_words(int rows, int n_part, int qcap) {
  return (size_t)kVqRows + (size_t)kVqRowStride * rows + (size_t)kVqSlotStride * n_part * qcap;
}

constexpr int kMaxGamma = 32;   // longest draft (positions per request)

// Temperature fit (sequential temperature scaling): one position k per
// pass.  hist holds n_bins x n_grid signed sums of (label - score) in 2^-30
// units (two's complement in 64 bits), bin-major; it lives in a buffer of
// the context that the passes leave zeroed.
// 16 waves per workgroup: occupancy without more workgroups, since each
// workgroup ends by adding its n_bins x n_grid sums into the global ones
constexpr int kStsThreads = 1024;
constexpr int kStsWaves = kStsThreads / 64;
constexpr int kStsMaxSlices = 4;                 // candidates per lane: n_grid <= 256
constexpr int kStsMaxGrid = 64 * kStsMaxSlices;
constexpr int kStsMaxBins = 64;
constexpr int kStsMaxCells = 4096;               // n_bins * n_grid (32 KB of LDS)

struct StsArgs {
  int64_t N;
  int gamma, k;                  // k: 1-based position fitted by this pass
  int n_grid, n_bins;
  int64_t stride;                // row stride of logit (elements)
  const float* logit;            // [N][stride]
  const int32_t* len;            // [N]
  const float* grid;             // [n_grid]
  float* T;                      // [gamma]: T[0 .. k-2] read, T[k-1] written
  int32_t* index;                // [gamma]
  double* ece;                   // [gamma][n_grid]
  unsigned long long* hist;      // [n_bins][n_grid], zero between positions
  unsigned int* done;            // workgroups finished in this pass, zero between passes
  int32_t* err;
};

struct ConfArgs {
  int B, gamma, V, dh, de;
  const uint16_t* h;
  const uint16_t* E;
  const int32_t* anchor;
  const int32_t* tokens;
  const uint16_t* wc;
  float bc;
  const float* sts;
  float* conf;
  float* surv;
  int32_t* err;
};

// The draft's merge of every position's chunk partials (CombineArgs) done by
// the confidence launch, a workgroup per request (dspark_draft_markov_conf).
struct ConfMergeArgs {
  CombineArgs m;
  ConfArgs f;
  unsigned int* cnt;             // [B] confidences formed per request, zero at launch and left zero
};

struct SchedArgs {
  int B, gamma, n_sps;
  const float* surv;
  const float* surv_hist;        // asynchronous rule: survivals two steps earlier
  const float* sps;
  int32_t* K;
  int32_t* n_selected;
  double* theta;
  uint64_t* sorted;              // [2][4096] keys by rank (set 1: current survivals, asynchronous rule)
};

// GRU head recurrence (position k: states[k] = GRU(states[k-1], W1[x_k])).
struct GruArgs {
  int B, R, V, k;
  const void* W1;                // [V][R], bf16 (w1_bf16) or fp32
  int w1_bf16;
  const uint16_t* W_ih;          // bf16 [3R][R], gate rows reset, update, new
  const uint16_t* W_hh;          // bf16 [3R][R]
  const uint16_t* b_ih;          // bf16 [3R]
  const uint16_t* b_hh;          // bf16 [3R]
  const uint16_t* s0;            // bf16 [R]
  const unsigned long long* best;   // running bests of position k: [kBestGroups][B]
  float* states;                 // fp32 [gamma][B][R]
  int32_t* err;
};

// Kernel lookup (host stubs usable with hipLaunchKernel and graph nodes).
// `wdtype`: 0 = fp32, 1 = bf16.  `depth` = D > 0: the workgroup-shared
// W2-tile variant walking `nt` 16-wide tiles per step and loading D steps
// ahead into LDS (bf16, r in {128, 256}; nt = 1 with D <= 3 or nt = 2 with
// D <= 2; grid = row-group quads x chunks); 0: the private-tile variant
// (grid = waves / 4).  `hs` = 1: the bias is projected from the fp32 GRU
// states in SweepArgs::hstate instead of W1 rows.  Returns nullptr if
// unsupported.
const void* sweep_kernel(int wdtype, int r, int mode, int depth, int nt, int hs);
// Whole-draft kernel (Markov head, bf16, r = 256, B <= 128, V <= 16 *
// kPersistTiles * waves): grid = one 256-thread workgroup per CU (plain or
// cooperative launch); n_vc = 4 * grid.  nullptr for other modes.
constexpr int kPersistTiles = 10;
const void* draft_persist_kernel(int mode);
// Chained draft (Markov head, bf16, B <= 128, r in {128, 256}): every
// position in one launch of persistent workgroups of `waves` waves claiming
// (position, request group, chunk) items in order; a group is waves x
// rows_per_wave requests.  Shapes (waves, rows_per_wave, depth, nt): (4, 32,
// 1, 2) and (4, 32, 2, 1) for r = 256, (4, 32, 1, 2) for r = 128; (4, 16, 1,
// 2) for both; (8, 16, 2..4, 2) for r = 256, (8, 16, 2, 2) for r = 128.
// nullptr otherwise.
const void* draft_chain_kernel(int r, int mode, int depth, int nt, int rows_per_wave, int waves);
constexpr int kChainMaxGrid = 2048;   // workgroups of a chained draft launch (release flags)
const void* combine_draft_kernel();
const void* combine_resid_kernel();
const void* combine_alpha_kernel();
const void* rows_lse_kernel();
const void* verify_rows_kernel();
const void* verify_decide_kernel();
const void* verify_chain_kernel();
const void* confidence_kernel();
const void* conf_merge_kernel();
// temperature fit: one scoring pass per position (its last workgroup selects)
const void* sts_hist_kernel(int n_slices, int cells);   // 1..4 slices of 64 candidates per lane
const void* gru_init_kernel();
const void* gru_step_kernel(int r);
int gru_step_threads(int r);   // workgroup size of gru_step_kernel(r)
const void* schedule_kernel(int async);
const void* schedule_rank_kernel();

constexpr int kSchedMaxKeys = 8192;
constexpr int kSchedThreads = 1024;

// Streaming-read calibration (stream.hip): the sum of n floats (x 16-byte
// aligned), per-workgroup partials, then one workgroup sums them in order.
struct StreamArgs {
  const float* x;
  int64_t n, n4;                 // floats, whole float4s
  float* partials;               // [grid] of the read pass
  int n_part;
  float* out;
};
constexpr int kStreamThreads = 256;
const void* stream_read_kernel();
const void* stream_sum_kernel();

}  // namespace dspark
