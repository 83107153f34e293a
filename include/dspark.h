/*
 * libdspark -- the per-step draft/verify hot path of DSpark's
 * confidence-scheduled speculative decoding, for AMD Instinct MI355X (gfx950).
 *
 * Pages cited (by title and section):
 *   [blog]     "DSpark：半自回归生成与置信度调度的投机解码"
 *              (pinghaoyang.com.cn/aigc/posts/dspark/)
 *   [teardown] "拒绝盲猜与算力空转：深度拆解 DeepSeek 开源投机采样方案 DeepSpec & DSpark"
 *              (val213.github.io/2026/06/28/DSpark&DSpec/)
 *   [summary]  "DeepSeek-AI与北京大学联手破局：AI聊天机器人'慢速打字'的终极解决方案"
 *              (techwalker.com/2026/0716/3193540.shtml)
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Every tensor argument is a device pointer to caller-owned memory on the
 *    context's device.  The library never frees, keeps or reallocates it.
 *  - Calls are asynchronous on `stream`: they enqueue kernels and return.
 *    Outputs are valid once the stream reaches the call.  Calls on one
 *    context must not run concurrently on different streams (the context's
 *    workspace is shared); a context is used by one host thread at a time.
 *  - The calls enqueue kernels only (no memset, no host synchronisation once
 *    the context's workspace has grown to the shape), so a caller may capture
 *    them into a HIP graph after one call of the same shapes on the context;
 *    a replay re-runs the captured arguments (pointers, seed).  Neither the
 *    cooperative launch of the whole-draft kernel (the default for small
 *    batches: capture those with DSPARK_PERSIST=0, or DSPARK_PERSIST_COOP=0
 *    on an otherwise idle device) nor the library's own graph of the draft
 *    loop (DSPARK_GRAPH=1) is meant for capture.
 *  - Row-major layouts; strides are in elements.  Logit rows (U, target) are
 *    contiguous over the vocabulary and 16-byte aligned.
 *  - Tokens and request ids are 32-bit.  Request ids are read as unsigned.
 *  - Random numbers come from a counter-based hash keyed on
 *    (seed, request id, 1-based position, purpose): SplitMix64's output
 *    function builds the 64-bit row key, MurmurHash3's fmix32 mixes each
 *    vocabulary index, u = (2*(h>>9)+1)*2^-24.  Results are therefore a
 *    deterministic function of the inputs and the seed (bitwise repeatable).
 *  - temperature == 0 selects greedy (argmax) drafting and verification.
 *  - Return codes: DSPARK_OK, or DSPARK_EINVAL (bad argument, checked on the
 *    host before anything is enqueued), DSPARK_EHIP (a HIP call failed),
 *    DSPARK_ENOMEM (workspace could not grow).  The message is available
 *    from dspark_last_error.  Kernels that meet an out-of-range token id or
 *    verify length clamp it and raise a device error flag, reported as
 *    DSPARK_EDEVICE by dspark_check.
 *  - Tracing: with DSPARK_ROCTX=1 in the environment when the library makes
 *    its first call, every call below (and dspark_check) is a named host
 *    range in a profiler's marker trace (roctx, loaded at run time; e.g.
 *    rocprofv3 --marker-trace).  Without it nothing is loaded.
 */
#ifndef DSPARK_H
#define DSPARK_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct dspark_ctx dspark_ctx;

enum {
  DSPARK_OK = 0,
  DSPARK_EINVAL = 1,
  DSPARK_EHIP = 2,
  DSPARK_ENOMEM = 3,
  DSPARK_EDEVICE = 4
};

/* Weight element types of the Markov head. */
typedef enum { DSPARK_F32 = 0, DSPARK_BF16 = 1 } dspark_dtype;

/* Library ABI version (major * 100 + minor). */
int dspark_version(void);

/* Create a context bound to HIP device `device`.  It owns a growable device
 * workspace (cross-block partial results, scheduler scratch), a cache of
 * instantiated HIP graphs for the draft loop (used when the environment sets
 * DSPARK_GRAPH=1; by default the loop is launched kernel by kernel, which
 * leaves no idle gap after the loop), and a device error flag.
 * Returns DSPARK_EINVAL for a null `out`, DSPARK_EHIP if the device cannot be
 * used.  On failure *out is set to NULL. */
int dspark_create(dspark_ctx** out, int device);

/* Release everything the context owns.  Waits for the device first.  NULL is
 * accepted. */
void dspark_destroy(dspark_ctx* ctx);

/* Message of the last failing call on this context ("" if none).  The
 * pointer stays valid until the next call on the context. */
const char* dspark_last_error(const dspark_ctx* ctx);

/* Synchronise `stream`, read and clear the device error flag.  Returns
 * DSPARK_EDEVICE if any kernel since the last check met an out-of-range
 * token id, verify length or accepted length, a bad candidate temperature
 * (dspark_sts_fit), or a grid barrier of the whole-draft kernel
 * gave up waiting (see dspark_draft_markov; the message names which),
 * DSPARK_EHIP on a HIP error, else DSPARK_OK. */
int dspark_check(dspark_ctx* ctx, hipStream_t stream);

/* Kernel timing for benchmarks (not needed for correct use).
 * While enabled, every kernel the context launches carries a start and a
 * stop HIP event attached to its dispatch (they bracket the kernel's
 * execution, not the queue's ordering gap before it; a cooperative launch of
 * the whole-draft kernel, the default for small batches, is bracketed by events
 * recorded on the stream around it instead, which include that gap), and
 * the draft loop is
 * launched kernel by kernel even where a graph was requested.  dspark_timing_read waits
 * for the recorded events, writes per-kernel-class totals (milliseconds) and
 * launch counts into arrays of DSPARK_K_COUNT entries, and forgets them.
 * Errors: DSPARK_EINVAL for null arguments, DSPARK_EHIP if an event fails. */
enum {
  DSPARK_K_DRAFT_SWEEP = 0,    /* MFMA bias + vocabulary sweep of one position (or of
                                  every position: the whole-draft kernel) */
  DSPARK_K_DRAFT_COMBINE = 1,  /* cross-chunk merge of one position */
  DSPARK_K_CONFIDENCE = 2,     /* confidences and survival products (one launch) */
  DSPARK_K_SURVIVAL = 3,       /* kept for numbering; nothing is launched in it */
  DSPARK_K_SCHEDULE = 4,
  DSPARK_K_VERIFY_ROWS = 5,    /* streaming pass over target rows */
  DSPARK_K_VERIFY_DECIDE = 6,  /* per-request merge of its rows + accept tests */
  DSPARK_K_RESID_SWEEP = 7,    /* MFMA residual sweep */
  DSPARK_K_RESID_COMBINE = 8,
  DSPARK_K_GRU = 9,            /* GRU head: s_0 fill and state updates */
  DSPARK_K_DIAG = 10,          /* diagnostic passes (dspark_accept_prob) */
  DSPARK_K_STS = 11,           /* temperature fit: the pass of one position */
  DSPARK_K_DRAFT_CHAIN = 12,   /* chained draft: every position in one launch */
  DSPARK_K_VERIFY_CHAIN = 13,  /* verify chain: every needed target row in one launch */
  DSPARK_K_CONF_MERGE = 14,    /* draft merge + confidences (dspark_draft_markov_conf) */
  DSPARK_K_COUNT = 15
};
int dspark_timing_enable(dspark_ctx* ctx, int enable);
int dspark_timing_read(dspark_ctx* ctx, double* ms, int* launches);

/* Semi-autoregressive draft with the Markov head.
 *
 * [blog] "形式化定义", "整体架构" and "Markov Head：一阶转移偏置"; [teardown]
 * "DSpark 的解法": for k = 1..gamma and every request b,
 *     h      = W1[x_{k-1}]                 (x_0 = anchor[b])
 *     z_v    = U[b][k-1][v] + sum_i h_i * W2col_v[i]
 *     y_v    = z_v / T                     (T = temperature; y = z if T == 0)
 *     x_k    = argmin-index argmax_v z_v                     if T == 0
 *            = draw(exp(y), stream (seed, req_b, k, DRAFT))  else
 * where draw(w, s) is the Gumbel-max draw: the lowest v attaining
 * max_v (ln w_v - ln(-ln u_s(v))), so P(v) = w_v / sum w (u_s(v): the uniform of
 * element v of stream s).  x_k feeds position k+1.  Outputs per (b, k):
 *     tokens[b][k-1] = x_k
 *     lse[b][k-1]    = ln sum_v exp(y_v)      (of z when T == 0)
 *     ytok[b][k-1]   = y_{x_k}
 * so that ln p_d(x_k) = ytok - lse.
 *
 * B >= 1; 1 <= gamma <= 32; V >= 16, V % 16 == 0; r in {32, 64, 128, 256}.
 * U:      float rows of V logits at U + b*u_stride_b + (k-1)*u_stride_k,
 *         request-major ([B][>= gamma][V]: u_stride_k >= V, u_stride_b >=
 *         gamma*u_stride_k) or position-major ([>= gamma][B][V]: u_stride_b
 *         >= V, u_stride_k >= B*u_stride_b); strides are multiples of 4 and
 *         the pointer 16-byte aligned.
 * W1:     [V][r] row-major (token -> rank-r vector), dtype wdtype.
 * W2:     the r x V matrix W2 stored column-major, i.e. an array [V][r] whose
 *         row v is column v (an LM-head layout), dtype wdtype.  Both weight
 *         pointers 16-byte aligned.
 * anchor: int32 [B]; req_ids: uint32 [B] or NULL (then req = b).
 * tokens: int32 [B][gamma]; lse, ytok: float [B][gamma].
 * Logits must be finite.  Errors: DSPARK_EINVAL for shapes/pointers/
 * alignment/temperature < 0 or non-finite.
 *
 * Execution (every path computes the same function of the inputs: tokens
 * and ytok bit-identical, lse to rounding):
 *  - bf16 weights, r in {128, 256}, 65 <= B <= 128 (default): the chained
 *    draft, one launch for every position.  Persistent workgroups claim
 *    (position, vocabulary chunk) items from a ticket counter in position
 *    order; an item of position k starts streaming its U and W2 tiles, waits
 *    until every item of position k - 1 has published its chunk winners,
 *    then takes x_{k-1} and sweeps.  Items are claimed in dependency order
 *    by running workgroups, so the launch makes progress however many of its
 *    workgroups are resident (concurrent kernels on other streams only slow
 *    it down).  Its waits are bounded all the same (about a second): a wait
 *    that gives up lets the item run on, the results are invalid and
 *    dspark_check reports DSPARK_EDEVICE.  DSPARK_CHAIN=0 selects the
 *    per-position sweeps instead.
 *  - bf16 weights, r = 256, B <= 48 (default) and V <= 16 * 10 * 4 * (compute
 *    units): the whole-draft kernel, one launch of one workgroup per compute
 *    unit that keeps W2 in registers and separates positions with a grid
 *    barrier.  Its workgroups must all be resident to pass a barrier, so by
 *    default it is launched cooperatively (co-residency guaranteed by the
 *    runtime, also when other streams run kernels; ~20-25 us more per
 *    call).  When the runtime refuses the cooperative launch (it does while
 *    another process on the device holds its cooperative-launch resource),
 *    that call runs on the per-position sweeps instead, with the same
 *    greedy tokens; the next call tries the whole-draft kernel again.
 *    DSPARK_PERSIST_COOP=0 launches it plainly, for callers that own an
 *    otherwise idle device: there, if concurrent kernels hold compute units,
 *    the waiting workgroups start as those kernels finish, and two such
 *    launches at once can wait for each other until the bounded barrier
 *    gives up (DSPARK_EDEVICE from dspark_check).  DSPARK_PERSIST=0 never
 *    uses this kernel, =2 uses it for every eligible batch up to 128
 *    requests (ahead of the chained draft).
 *  - otherwise: one vocabulary sweep per position, each taking x_{k-1} from
 *    the previous sweep, then one merge.
 * Environment variables are read when the context is created. */
int dspark_draft_markov(dspark_ctx* ctx, hipStream_t stream,
                        int B, int gamma, int V, int r, dspark_dtype wdtype,
                        const float* U, int64_t u_stride_b, int64_t u_stride_k,
                        const void* W1, const void* W2,
                        const int32_t* anchor, const uint32_t* req_ids,
                        float temperature, uint64_t seed,
                        int32_t* tokens, float* lse, float* ytok);

/* Allocation-free variant of dspark_draft_markov, for callers that cannot
 * allocate: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments, same results (bit-identical tokens,
 * lse and ytok) as dspark_draft_markov with the same context settings, except
 * that it never uses the whole-draft kernel (small batches run the
 * per-position sweeps).  Its partials, running-best slot groups and
 * chained-draft counters live in one file-scope device array of 16 MiB per
 * GPU (held until the process ends), whose device address is taken once per
 * device when a context is created there; the call allocates nothing, creates
 * no event or graph and launches its kernels directly (the context's timing
 * and graph switches are ignored).  Limits: B * n_chunks * gamma * 24 bytes
 * of partials within 15,040 KiB (on a 256-CU part the chained draft cuts
 * the vocabulary into 256 chunks: the headline shape B = 128, gamma = 7,
 * V = 151936 needs 5,376 KiB, and gamma <= 19 fits at B = 128) and
 * B * gamma <= 8192;
 * a larger shape returns DSPARK_EINVAL with the sizes in the message.
 * Every call on a GPU, from any context, shares that GPU's array: calls that
 * overlap on one GPU (other streams, other threads) race and must be
 * serialised by the caller.  Each call leaves the array's slot groups and
 * counters zero for the next one.  DSPARK_EHIP if the array's address could
 * not be taken when the context was created. */
int dspark_draft_markov_static(dspark_ctx* ctx, hipStream_t stream,
                               int B, int gamma, int V, int r, dspark_dtype wdtype,
                               const float* U, int64_t u_stride_b, int64_t u_stride_k,
                               const void* W1, const void* W2,
                               const int32_t* anchor, const uint32_t* req_ids,
                               float temperature, uint64_t seed,
                               int32_t* tokens, float* lse, float* ytok);

/* Semi-autoregressive draft with the RNN (GRU) head.
 *
 * [blog] "RNN Head：长程依赖"; [summary] section 3 (the state-vector head).
 * As dspark_draft_markov, except that the bias of position k is projected
 * from a recurrent state instead of the previous token's W1 row:
 *     s_0    = s0                          (learned, the same for every request)
 *     z_v    = U[b][k-1][v] + sum_i s_{k-1}[i] * W2col_v[i]
 *     s_k    = GRU(s_{k-1}, W1[x_k])       (k < gamma)
 * with the textbook GRU cell, gate rows in the order reset, update, new:
 *     r  = sigmoid(W_ih[0:r] x + b_ih[0:r] + W_hh[0:r] s + b_hh[0:r])
 *     z  = sigmoid(W_ih[r:2r] x + b_ih[r:2r] + W_hh[r:2r] s + b_hh[r:2r])
 *     n  = tanh(W_ih[2r:3r] x + b_ih[2r:3r] + r * (W_hh[2r:3r] s + b_hh[2r:3r]))
 *     s' = (1 - z) * n + z * s
 * The state is carried in fp32 (it enters the bf16 MFMA projection as a
 * hi + lo pair, so the bias is fp32-accurate).  The anchor token does not
 * enter.  Inputs as for dspark_draft_markov, plus W_ih, W_hh: bf16 [3r][r]
 * (16-byte aligned); b_ih, b_hh: bf16 [3r]; s0: bf16 [r].
 * states: float [gamma][B][r], 16-byte aligned: states[k-1][b] is the state
 * position k projected (s_0 .. s_{gamma-1}); pass it to dspark_verify. */
int dspark_draft_rnn(dspark_ctx* ctx, hipStream_t stream,
                     int B, int gamma, int V, int r, dspark_dtype wdtype,
                     const float* U, int64_t u_stride_b, int64_t u_stride_k,
                     const void* W1, const void* W2,
                     const void* W_ih, const void* W_hh, const void* b_ih,
                     const void* b_hh, const void* s0,
                     const uint32_t* req_ids, float temperature, uint64_t seed,
                     int32_t* tokens, float* lse, float* ytok, float* states);

/* Confidence head with sequential temperature scaling and survival products.
 *
 * [blog] "置信度头：预测自己的命运" and "校准问题：原始置信度不可靠"; [summary]
 * section 4; [teardown] "硬件感知前缀调度器" (survival product):
 *     l_k   = sum_i wc[i] h[b][k-1][i] + sum_j wc[d_h + j] E[x_{k-1}][j] + bc
 *     c_k   = 1 / (1 + exp(-l_k / T_k))        (T_k = sts_T[k-1], or 1)
 *     a_k   = c_1 * c_2 * ... * c_k
 * with x_0 = anchor[b], x_k = tokens[b][k-1].
 * h: bf16 [B][gamma][d_h]; E: bf16 [V][d_e]; wc: bf16 [d_h + d_e];
 * d_h, d_e multiples of 8, >= 8; h, E, wc 16-byte aligned.
 * sts_T: float [gamma] or NULL; conf, surv: float [B][gamma]. */
int dspark_confidence(dspark_ctx* ctx, hipStream_t stream,
                      int B, int gamma, int V, int d_h, int d_e,
                      const void* h, const void* E,
                      const int32_t* anchor, const int32_t* tokens,
                      const void* wc, float bc, const float* sts_T,
                      float* conf, float* surv);

/* Markov-head draft followed by the confidence head, in fewer launches.
 *
 * The same results as dspark_draft_markov (tokens, lse, ytok, bit for bit)
 * then dspark_confidence on those tokens (conf, surv, bit for bit), with the
 * draft's merge of its chunk partials done by the confidence launch: one
 * workgroup per (request, position k) merges position k in the draft
 * combine's order and forms the confidence whose previous token is x_k
 * (c_{k+1}; c_1 from the anchor in the workgroup of k = gamma), and the
 * last of a request's workgroups to finish forms its survival products.
 * One launch fewer per step.  Arguments: those of dspark_draft_markov, then
 * d_h, d_e, h, E, wc, bc, sts_T as for dspark_confidence, then the outputs
 * of both; the limits and errors of both apply.  The context keeps a block
 * of per-request counters (allocated on the first call with a batch larger
 * than any before, left at zero by every call), so calls that overlap on
 * one context race, as for the draft's own workspace. */
int dspark_draft_markov_conf(dspark_ctx* ctx, hipStream_t stream,
                             int B, int gamma, int V, int r, dspark_dtype wdtype,
                             const float* U, int64_t u_stride_b, int64_t u_stride_k,
                             const void* W1, const void* W2, const int32_t* anchor,
                             const uint32_t* req_ids, float temperature, uint64_t seed,
                             int d_h, int d_e, const void* h, const void* E,
                             const void* wc, float bc, const float* sts_T,
                             int32_t* tokens, float* lse, float* ytok,
                             float* conf, float* surv);

/* Hardware-aware prefix scheduler: greedy admission with early stop.
 *
 * [blog] "硬件感知前缀调度器" (steps 1-4); [summary] sections 4-5.  All (b, j)
 * candidates are sorted by (surv[b][j-1] descending, b ascending, j
 * ascending) and admitted one at a time; after admitting n of them
 *     Theta_n = (B + S_n) * sps[B + n - 1],   S_n = sum of admitted survivals,
 *     Theta_0 = B * sps[B - 1];
 * admission stops at the first n with Theta_n <= Theta_{n-1} or with
 * B + n > n_sps.  K[b] = number of admitted candidates of request b (always
 * a prefix 1..K[b]).  Sums and Theta are formed in float64.
 * surv: float [B][gamma], values in [0, 1] (non-finite or negative read as
 * 0); sps: float [n_sps], sps[N-1] the verify steps/s at N tokens.
 * 1 <= B <= n_sps; B * gamma <= 4096.
 * K: int32 [B]; n_selected: int32 [1]; theta: double [1] (Theta at the
 * admitted set). */
int dspark_schedule(dspark_ctx* ctx, hipStream_t stream,
                    int B, int gamma, const float* surv,
                    const float* sps, int n_sps,
                    int32_t* K, int32_t* n_selected, double* theta);

/* Asynchronous prefix scheduler: capacity from history, order from now.
 *
 * [blog] "硬件感知前缀调度器" (the asynchronous mechanism: the verify length
 * is estimated from the confidences of earlier steps so scheduling does not
 * stall the pipeline); [summary] section 5 (the production rule: the count
 * comes from confidences two steps old, candidates are still ranked by the
 * latest ones, and the early-stop break is replaced by a global search).
 *     Theta_n = (B + S_n) * sps[B + n - 1],  S_n = sum of the n largest
 *               surv_hist values,  Theta_0 = B * sps[B - 1],
 *     n*      = the first n attaining max Theta_n, 0 <= n <= min(B*gamma,
 *               n_sps - B)  (no early stop),
 * then the top n* candidates of surv, sorted (surv descending, b ascending,
 * j ascending), are admitted: K[b] = their count for request b (a prefix).
 * theta receives Theta_{n*}.  surv_hist: float [B][gamma], the same request
 * slots two steps earlier (same value rules as surv).  Other arguments and
 * limits as for dspark_schedule. */
int dspark_schedule_async(dspark_ctx* ctx, hipStream_t stream,
                          int B, int gamma, const float* surv,
                          const float* surv_hist, const float* sps, int n_sps,
                          int32_t* K, int32_t* n_selected, double* theta);

/* Lossless speculative verification with residual resampling and a bonus.
 *
 * [blog] "形式化定义"; [summary] sections 1 and 4.  For request b with verify
 * length K_b (K[b], or gamma if K is NULL), positions k = 1..K_b in order:
 *     T == 0: keep x_k iff x_k == argmin-index argmax_v target[b][k-1][v];
 *             otherwise emit that argmax and stop.
 *     T  > 0: p_t = softmax(target[b][k-1] / T), p_d from the draft
 *             (ln p_d(x_k) = ytok - lse); keep x_k iff
 *             u(seed, req_b, k, ACCEPT, 0) < p_t(x_k) / p_d(x_k);
 *             at the first rejection emit draw(r, stream (seed, req_b, k,
 *             RESID)), r_v = max(0, p_t(v) - p_d(v)), recomputing the draft
 *             row from U, W2 and either W1 + anchor (Markov head) or states
 *             (GRU head: the bias at position k is states[k-1][b] . W2); if
 *             every r_v is 0, draw(p_t) with the same stream; draw() as for
 *             dspark_draft_markov.
 * If all K_b drafts are kept, emit the bonus token from target row K_b + 1
 * (its argmax, or draw(exp(t / T)) with purpose BONUS at position K_b+1).
 * Outputs: accept_len[b] = number kept; out_tokens[b][0..accept_len] = the
 * kept drafts followed by the emitted token, then -1 up to gamma.
 * target: float [B][>= gamma+1][V] (same stride rules as U).  The other
 * arguments are those given to / returned by dspark_draft_markov, or by
 * dspark_draft_rnn (states non-NULL; W1 and anchor may then be NULL); K:
 * int32 [B] or NULL (values outside 0..gamma are clamped and flagged).
 * accept_len: int32 [B]; out_tokens: int32 [B][gamma+1].
 * Execution: target rows after a request's first rejection are not read.
 * By default the rows are read in windows (rows 1-2 of every request, then
 * rows 3-4, then the rest, of the requests that kept every draft so far),
 * each a row pass and a decision launch (DSPARK_VERIFY_WINDOWS="e1,e2,..."
 * sets the last row of each window but the final one).  DSPARK_VERIFY_CHAIN=1 reads every
 * needed row in one launch instead, deciding each request row by row as its
 * rows complete (rows read DSPARK_VERIFY_AHEAD ahead, default 2; V up to
 * 524288); the outputs are identical. */
int dspark_verify(dspark_ctx* ctx, hipStream_t stream,
                  int B, int gamma, int V, int r, dspark_dtype wdtype,
                  const float* target, int64_t t_stride_b, int64_t t_stride_k,
                  const float* U, int64_t u_stride_b, int64_t u_stride_k,
                  const void* W1, const void* W2, const int32_t* anchor,
                  const int32_t* tokens, const float* lse, const float* ytok,
                  const float* states, const int32_t* K, const uint32_t* req_ids,
                  float temperature, uint64_t seed,
                  int32_t* accept_len, int32_t* out_tokens);

/* Diagnostics: per-position acceptance probabilities.
 *
 * [summary] section 4 (the confidence head is trained toward the true
 * acceptance rate, the total-variation distance between the draft and the
 * target distributions) and [blog] "置信度头" (c_k is P(position k accepted |
 * the earlier ones were)).  Under the lossless rule the drafted token at
 * position k is kept with probability
 *     alpha[b][k-1] = sum_v min(p_d(v), p_t(v)) = 1 - TV(p_d, p_t)
 * given its prefix, p_d the draft law (U and the bias of the head that
 * drafted: W1 + anchor + tokens for the Markov head, states for the GRU
 * head), p_t = softmax(target[b][k-1] / T).  Averaged over requests it
 * gives the acceptance curve per position.  A diagnostic pass outside the
 * step: it reads every target row 1..gamma and rebuilds every draft row.
 * Arguments as for dspark_verify (target needs only gamma rows);
 * temperature > 0; alpha: float [B][gamma]. */
int dspark_accept_prob(dspark_ctx* ctx, hipStream_t stream,
                       int B, int gamma, int V, int r, dspark_dtype wdtype,
                       const float* target, int64_t t_stride_b, int64_t t_stride_k,
                       const float* U, int64_t u_stride_b, int64_t u_stride_k,
                       const void* W1, const void* W2, const int32_t* anchor,
                       const int32_t* tokens, const float* lse, const float* states,
                       float temperature, float* alpha);

/* Lossless verification over a flattened (packed) target.
 *
 * [summary] section 5 (the variable-length verify batch: every request's
 * rows to verify are laid end to end and a marker / offset tensor records
 * which request and position each row belongs to).  As dspark_verify, but
 * the target rows of request b, positions 1 .. K[b] + 1, are rows
 * t_offsets[b] .. t_offsets[b] + K[b] of a packed float array of n_rows
 * rows, row stride t_row_stride (>= V, multiple of 4; 16-byte aligned
 * pointer): no padding rows are stored for positions past K[b] + 1.  K is
 * required.  A row index outside [0, n_rows) is flagged (reported by
 * dspark_check as a packed-row error) and replaced by row 0. */
int dspark_verify_packed(dspark_ctx* ctx, hipStream_t stream,
                         int B, int gamma, int V, int r, dspark_dtype wdtype,
                         const float* target, int64_t t_row_stride,
                         const int32_t* t_offsets, int n_rows,
                         const float* U, int64_t u_stride_b, int64_t u_stride_k,
                         const void* W1, const void* W2, const int32_t* anchor,
                         const int32_t* tokens, const float* lse, const float* ytok,
                         const float* states, const int32_t* K, const uint32_t* req_ids,
                         float temperature, uint64_t seed,
                         int32_t* accept_len, int32_t* out_tokens);

/* Fit the per-position confidence temperatures (sequential temperature
 * scaling) on held-out drafts.
 *
 * [blog] "校准问题：原始置信度不可靠" and [summary] section 4: for k = 1 ..
 * gamma in order, T_k is the candidate temperature whose calibrated survival
 *     S_n(T) = prod_{i<k} sigmoid(l[n][i] / T_i) * sigmoid(l[n][k-1] / T)
 * has the lowest expected calibration error against the labels
 * y_n = [accept_len[n] >= k] (the first k drafted tokens of sample n were
 * accepted); T_1 .. T_{k-1} are the temperatures already fitted.  The error
 * is the binned one with n_bins equal-width bins on [0, 1] (sample n in bin
 * min(floor(S_n n_bins), n_bins - 1)):
 *     ECE = sum over bins of (n_m / N) |mean label - mean score|
 *         = sum over bins of |sum_{n in bin} (y_n - S_n)| / N,
 * and 0 when N == 0.  Ties go to the lowest candidate index.  The result is
 * what dspark_confidence takes as sts_T.
 *
 * 0 <= N < 2^33 samples (a cell's sum of |label - score| in 2^-30 units
 * then stays below 2^63); 1 <= gamma <= 32.
 * logit:      float [N][stride] (stride >= gamma): the confidence head's
 *             logits l = logit(c) before any temperature, positions 1..gamma
 *             in columns 0..gamma-1.  May be NULL when N == 0.
 * accept_len: int32 [N], accepted draft lengths in 0..gamma (verification
 *             of all gamma positions).  May be NULL when N == 0.
 * grid:       float [n_grid] candidate temperatures, each positive and
 *             finite; 1 <= n_grid <= 256, 1 <= n_bins <= 64,
 *             n_grid * n_bins <= 4096.
 * T:          float [gamma] out: the fitted temperatures (values of grid).
 * index:      int32 [gamma] out: their indices in grid.
 * ece:        double [gamma][n_grid] out: the error of every candidate at
 *             every position (given the earlier fitted temperatures).
 * Arithmetic: scores in fp32 (hardware exponential and reciprocal); each
 * sum of (y - S) is accumulated exactly as an integer of 2^-30 units
 * (per-sample truncation), so results do not depend on the order in which
 * the workgroups finish.  A score within a few fp32 ulps of a bin edge may
 * fall in the neighbouring bin of an exact evaluation.
 * Tuning: DSPARK_STS_WG_PER_CU (1..16, default 2) sets the workgroups of a
 * pass per CU; it does not change results.
 * Errors: DSPARK_EINVAL for shapes, limits and null pointers; DSPARK_ENOMEM
 * if the context's 33 KB buffer for the sums (allocated at its first fit)
 * cannot be allocated.  A candidate that is not positive and finite or an
 * accepted length outside [0, gamma] (clamped) raises the device error flag
 * (dspark_check).  Launches gamma kernels, one per position (timing class
 * DSPARK_K_STS); the last workgroup of each selects its temperature. */
int dspark_sts_fit(dspark_ctx* ctx, hipStream_t stream, int64_t N, int gamma,
                   const float* logit, int64_t stride, const int32_t* accept_len,
                   const float* grid, int n_grid, int n_bins,
                   float* T, int32_t* index, double* ece);

/* Streaming-read calibration (measurement support, not part of decoding).
 *
 * For benchmarks that relate the path's streaming kernels to what a plain
 * read reaches on the device: out[0] = the float32 sum of x[0 .. n), every
 * element read once in 16-byte loads (per-workgroup partials, then one
 * workgroup adds them in a fixed order, so the result is the same on every
 * call with the same n and device).  Timed over a buffer larger than the
 * last-level cache it gives the read bandwidth the memory sustains.
 *
 * x: device, 16-byte aligned, n >= 0 floats (n = 0 writes 0); out: device,
 * one float.  Uses the context's workspace for one float per workgroup.
 * Two launches (timing class DSPARK_K_DIAG).  Errors: DSPARK_EINVAL for a
 * null or misaligned pointer or n < 0; DSPARK_ENOMEM, DSPARK_EHIP as for
 * the other calls. */
int dspark_stream_read(dspark_ctx* ctx, hipStream_t stream, const float* x, int64_t n, float* out);

#ifdef __cplusplus
}
#endif

#endif /* DSPARK_H */
