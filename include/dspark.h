/*
 * dspark.h - C ABI of the DSpark draft / verify / confidence hot path on gfx950.
 *
 * Pages cited (titles as published):
 *   [P1] "大模型推理加速的系统级工程：DeepSeek V4-Pro DSpark 推测解码方案深度解析与开源工具链
 *        DeepSpec" (Best Partners TV, 2026-06-30)
 *   [P2] "DeepSeek 开源 DSpark，一个可将大语言模型推理速度提升高达 85% 的新框架" (VentureBeat,
 *        Chinese translation)
 *   [P3] "DSpark Speculative Decoding" (concept note)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Memory     Every array argument is DEVICE memory owned by the caller, row-major with the
 *            last dimension contiguous. The library allocates nothing: scratch comes from
 *            the caller's workspace `ws` of at least `dspark_*_workspace_bytes(...)` bytes
 *            (256-byte aligned, as the HIP allocator returns). Its contents need no
 *            preparation; a call owns it until the call's work on `stream` has finished, so
 *            calls that may overlap need distinct workspaces. (The one-launch draft forms
 *            keep a call counter in the workspace and reset their own position slots
 *            inside the launch; any bytes, including those of other calls, are accepted.)
 * Streams    `stream` is a hipStream_t (NULL = the null stream). Calls only enqueue work and
 *            return without synchronising. Calls on distinct workspaces may run concurrently;
 *            the library keeps no mutable global state.
 * Errors     Every call returns a status. Host-detected errors (bad sizes, NULL required
 *            pointers, a workspace that is too small, caps exceeded) enqueue nothing and leave
 *            all outputs untouched. DSPARK_ERR_HIP reports a failed kernel launch.
 *            dspark_last_error() returns a per-thread text describing the last failure.
 * Device     Faults in device-resident data cannot be reported synchronously; they produce
 * data       sentinels instead: a token id outside [0, V) gives token -1 (and n = -1 in
 *            verify), a logit row that is entirely -inf gives token -1, uniforms are clamped
 *            into [0, 1 - 2^-24]. NaN logits are undefined behaviour.
 * Dtypes     Logits, uniforms, confidences and speeds are fp32; tokens, lengths and offsets
 *            are int32. Markov factors are fp32 (DSPARK_F32) or bf16 (DSPARK_BF16).
 * Sampling   One host uniform per draw; the token is the inverse CDF in token-id order,
 *            x = min { v : F(v) > u }.
 * Caps       1 <= B <= 2^24; 1 <= gamma <= 64; 1 <= r <= 1024; 1 <= V < 2^31 with
 *            B*gamma*V < 2^40;
 *            scheduler R*gamma <= 16384 and R <= Bmax <= 2^20.
 * Results    Deterministic: two calls on the same inputs give bit-identical outputs (no float
 *            atomics; every reduction has a fixed order or is an exact integer sum).
 */
#ifndef DSPARK_H
#define DSPARK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    DSPARK_OK = 0,
    DSPARK_ERR_INVALID_ARG = 1,
    DSPARK_ERR_WORKSPACE = 2,
    DSPARK_ERR_UNSUPPORTED = 3,
    DSPARK_ERR_HIP = 4
};

enum { DSPARK_F32 = 0, DSPARK_BF16 = 1 };

enum { DSPARK_SCHED_GLOBAL = 0, DSPARK_SCHED_EARLY_STOP = 1 };

/* Static text of a status code. */
const char* dspark_status_string(int status);

/* Per-thread description of the last non-OK status returned on this thread ("" if none). */
const char* dspark_last_error(void);

/* ABI version: major * 10000 + minor * 100 + patch. */
int dspark_version(void);

/*
 * Markov-head sequential draft.
 * [P3] "Semi-Autoregressive Generation": x_k ~ p_k(v) proportional to exp(U_k(v) + B_k(v))
 * with the low-rank Markov bias B_k = W1[x_{k-1}] W2 (rank r); [P1] section
 * "DSpark 架构设计：半自回归生成与马尔可夫修正": the head conditions only on the previous token
 * and runs left to right. Position 1 conditions on the context token x0.
 *
 *   U       [B][gamma][V]  fp32 base logits from the parallel backbone (read only)
 *   W1      [V][r]         Markov factor, dtype w_dtype (read only)
 *   W2      [r][V]         Markov factor, dtype w_dtype (read only)
 *   x0      [B]            int32 last committed token of each request
 *   u       [B][gamma]     fp32 host uniforms, one per draw
 *   x_out   [B][gamma]     int32 draft tokens (required)
 *   q_out   [B][gamma]     fp32 p_k(x_k)                      (nullable)
 *   lse_out [B][gamma]     fp32 logsumexp(U_k + B_k)          (nullable)
 *   Ld_out  [B][gamma][V]  fp32 draft logits U_k + B_k        (nullable)
 * Positions run in order on `stream` without host round trips. Four kernel paths compute
 * this same function (dspark_markov_draft_path tells which one a call takes); each is
 * deterministic, and they differ from one another only in fp32 rounding order:
 *   DSPARK_PATH_SWEEP     one vocabulary sweep per position (B <= 8, or fp32 factors).
 *   DSPARK_PATH_SLAB      every workgroup keeps its vocabulary slab of W2 in registers as
 *                         bf16 MFMA operands and streams the batch through it; the draw
 *                         recomputes the chosen tile's logits instead of reading them (B > 8,
 *                         bf16, r <= 256 and r % 8 == 0, V % 8 == 0, V <= 163840, B <= 2048
 *                         at V > 131072 and B <= 8192 at V > 98304, 16-byte aligned W1, W2,
 *                         U and Ld_out). Logits reach memory only when Ld_out is given.
 *                         Where the batch and every slab workgroup fit
 *                         (dspark_markov_draft_one_launch), all positions run in one launch
 *                         that holds W2 in registers throughout and separates positions by
 *                         flag barriers, with the same give-up behaviour and the same
 *                         restriction on overlapping draft calls as DSPARK_PATH_RESIDENT;
 *                         otherwise, or with DSPARK_DRAFT_PER_POSITION, each position is one
 *                         stream launch and one draw launch. Both forms draw the same tokens
 *                         and store the same logits bit for bit.
 *   DSPARK_PATH_MFMA      one bf16 MFMA projection per position (B > 8, bf16 factors, where
 *                         the slab path does not apply).
 *   DSPARK_PATH_RESIDENT  one launch for all positions, W2 held in registers across the GPU
 *                         (B = 1, bf16, r <= 256 and r % 8 == 0, V % 8 == 0, 16-byte aligned
 *                         factors, ceil(V / 640) <= compute units). Its workgroups must all be
 *                         resident at once: after every position each waits for the token
 *                         that all of their partial sums decide.
 *                         If other work keeps compute units busy for about a second, a
 *                         barrier gives up, and the positions not yet drawn get token -1,
 *                         q = 0 and lse = -inf. Draft calls on other streams of the same
 *                         device must not overlap a call that takes this path.
 */
enum { DSPARK_PATH_SWEEP = 0, DSPARK_PATH_MFMA = 1, DSPARK_PATH_RESIDENT = 2, DSPARK_PATH_SLAB = 3 };

/* The path dspark_markov_draft takes for these arguments on the current device, assuming a
 * 16-byte aligned U (and Ld_out) and no option bits; dspark_markov_draft_plan answers for the
 * exact call. */
int dspark_markov_draft_path(int B, int V, int r, int w_dtype, const void* W1, const void* W2);

/* 1 if dspark_markov_draft runs all positions in one launch for these arguments (a non-null
 * Ld_out when want_logits != 0), on the same assumptions as dspark_markov_draft_path. */
int dspark_markov_draft_one_launch(int B, int V, int r, int w_dtype, const void* W1, const void* W2,
                                   int want_logits);

/* Workspace of a draft call. dspark_markov_draft_workspace_bytes covers every path;
 * dspark_markov_draft_plan gives the exact call's path, whether it runs in one launch, and the
 * bytes that call needs (a call checks ws_bytes against that figure):
 *   single-request one-launch path   256 + slot bytes                  (kilobytes)
 *   slab path                        + 2 tile-partial buffers          (B * V / 16 bytes)
 *   sweep / MFMA without Ld_out      + 2 logits rows per request       (2 * B * V * 4 bytes)
 * Bytes 0..3 of the workspace hold, once a one-launch call has finished on its stream, a
 * give-up count (uint32): 0 when every position was drawn, nonzero when a wait gave up (the
 * positions not drawn then have token -1; the count may miss workgroups that gave up before
 * the launch reset the word, but never reads 0 after a give-up). Other paths leave the word
 * unchanged.
 * dspark_markov_draft_plan returns DSPARK_ERR_INVALID_ARG for arguments a call would reject as
 * sizes or dtypes; out pointers are host memory and nullable. */
size_t dspark_markov_draft_workspace_bytes(int B, int V, int r, int gamma);
int dspark_markov_draft_plan(int B, int V, int r, int gamma, int w_dtype, const void* W1,
                             const void* W2, const float* U, const float* Ld_out, int options,
                             int* path_out, int* one_launch_out, size_t* ws_bytes_out);
int dspark_markov_draft(int B, int V, int r, int gamma,
                        const float* U, const void* W1, const void* W2, int w_dtype,
                        const int32_t* x0, const float* u,
                        int32_t* x_out, float* q_out, float* lse_out, float* Ld_out,
                        void* ws, size_t ws_bytes, void* stream);

/* Option bits of dspark_markov_draft_ex.
 *   DSPARK_DRAFT_PER_POSITION  never the one-launch forms: every position is its own
 *                              launches (the slab path's stream + draw launches; a single
 *                              bf16 request takes DSPARK_PATH_SWEEP). The one-launch forms
 *                              hold every compute unit for the whole call; per-position
 *                              launches let kernels on other streams run between positions
 *                              and carry no restriction on overlapping draft calls. The
 *                              results are those of the one-launch form bit for bit on the
 *                              slab path, and equal to within fp32 rounding order otherwise. */
/*   DSPARK_DRAFT_TEST_SPIN     failure injection for tests: the one-launch forms poll each
 *                              wait once before giving up, so a wait that is not already
 *                              satisfied gives up (tokens -1 from that position on, the
 *                              workspace's give-up count set). Every kernel still exits. */
enum { DSPARK_DRAFT_PER_POSITION = 1, DSPARK_DRAFT_TEST_SPIN = 256 };

/* dspark_markov_draft with option bits (0 = dspark_markov_draft); unknown bits are
 * DSPARK_ERR_INVALID_ARG. Arguments, outputs and errors as dspark_markov_draft. */
int dspark_markov_draft_ex(int B, int V, int r, int gamma,
                           const float* U, const void* W1, const void* W2, int w_dtype,
                           const int32_t* x0, const float* u,
                           int32_t* x_out, float* q_out, float* lse_out, float* Ld_out,
                           void* ws, size_t ws_bytes, void* stream, int options);

/*
 * RNN-head sequential draft.
 * [P3] "Semi-Autoregressive Generation": the sequential stage samples x_k ~ p_k(v) proportional
 * to exp(U_k(v) + B_k(x_<k, v)); besides the default Markov head it names an RNN head that keeps
 * a recurrent state inside the block. [P1] section "DSpark 架构设计：半自回归生成与马尔可夫修正"
 * (the RNN head paragraph): an optional head whose hidden state, updated along the block,
 * carries longer-range dependence. The pages give no update rule; this library reads it as the
 * linear recurrence of the head's rank r
 *     h_1 = W1[x_0],  h_k = A h_{k-1} + W1[x_{k-1}],  B_k = h_k W2,
 * so that A = 0 is the Markov head (dspark_markov_draft, to fp32 rounding order).
 *
 *   U, W1, W2, x0, u, x_out, q_out, lse_out, Ld_out   as in dspark_markov_draft
 *   A       [r][r]         recurrence, dtype w_dtype (read only)
 *   h_out   [B][gamma][r]  fp32 state h_k each position's bias is formed from (nullable)
 * bf16 factors only (DSPARK_BF16; DSPARK_ERR_UNSUPPORTED otherwise), r <= 256 with r % 8 == 0,
 * V % 8 == 0, 16-byte aligned U, W1, W2 and A. The state is kept in fp32; the projection
 * multiplies its bf16 hi and lo parts (h = hi + lo to about 2^-17 relative) with W2 and
 * accumulates in fp32. Paths (dspark_rnn_draft_path): B = 1 where every workgroup fits runs
 * as DSPARK_PATH_RESIDENT (one launch, W2 in registers, A in LDS; the same give-up behaviour,
 * give-up word and restriction on overlapping draft calls); otherwise DSPARK_PATH_MFMA: one
 * launch for h_1, then two per position (the bf16 MFMA projection, whose extra workgroups
 * form A h_k meanwhile, and the draw, which adds the drawn token's W1 row). Sentinels as in
 * dspark_markov_draft; a dead request's state is 0.
 */
size_t dspark_rnn_draft_workspace_bytes(int B, int V, int r, int gamma);
int dspark_rnn_draft_path(int B, int V, int r, const void* W1, const void* W2, const void* A);
int dspark_rnn_draft(int B, int V, int r, int gamma,
                     const float* U, const void* W1, const void* W2, const void* A, int w_dtype,
                     const int32_t* x0, const float* u,
                     int32_t* x_out, float* q_out, float* lse_out, float* Ld_out, float* h_out,
                     void* ws, size_t ws_bytes, void* stream);

/*
 * Allocation-free draft, for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc). It is dspark_markov_draft_ex
 * with the workspace taken from a static device array of dspark_noalloc_scratch_bytes()
 * (32 MiB) that the library holds on each GPU it runs on until the process ends; it calls no
 * allocating routine. Arguments, outputs, paths and results are those of
 * dspark_markov_draft_ex bit for bit (the caller still passes inputs and outputs).
 * A call whose path needs more scratch than the array holds (dspark_markov_draft_plan's
 * ws_bytes; e.g. the sweep or MFMA path without Ld_out at large B * V) returns
 * DSPARK_ERR_UNSUPPORTED and enqueues nothing. Every call on one GPU shares that GPU's array
 * and finds the last call's bytes in it, which the draft accepts (its slots carry their own
 * call counter), so nothing needs clearing; calls that overlap on one GPU (other streams,
 * other threads) race on the array and must be ordered by the caller. The first call on a
 * device looks up the array's device address (hipGetSymbolAddress) with that device current;
 * a failure there returns DSPARK_ERR_HIP. The give-up word of a one-launch call is bytes 0..3
 * of the array.
 */
size_t dspark_noalloc_scratch_bytes(void);
int dspark_markov_draft_noalloc(int B, int V, int r, int gamma,
                                const float* U, const void* W1, const void* W2, int w_dtype,
                                const int32_t* x0, const float* u,
                                int32_t* x_out, float* q_out, float* lse_out, float* Ld_out,
                                void* stream, int options);

/*
 * Lossless rejection-sampling verification.
 * [P1] section "大模型推理的显存瓶颈与推测解码的演进逻辑" and [P3] intro: keep the longest accepted
 * prefix, resample at the first rejection, add a bonus token when all are kept. Rule (the
 * speculative sampling papers [P2] points to in "为什么推测解码很重要"): x_k is kept when
 * u_acc < p_t(x_k) / p_d(x_k) (tested as log u < log p_t(x) - log p_d(x); p_d(x) = 0 keeps iff
 * p_t(x) > 0); at the first rejection z ~ max(0, p_t - p_d) normalised (p_t if that mass is
 * zero); otherwise z ~ p_t at position len+1. [P1] section "极致的工程实现与内核优化": target
 * rows are flattened without padding.
 *
 *   Ld      [B][gamma][V]  fp32 draft logits (row k = position k+1)
 *   Lt      [Lt_rows][V]   fp32 flattened target logits: request b owns rows
 *                          t_off[b] .. t_off[b] + len[b]; row t_off[b] + i is position i+1
 *   Lt_rows                number of rows Lt holds (>= B*(gamma+1) when t_off is NULL)
 *   t_off   [B+1]          int32 row offsets (nullable: b * (gamma + 1))
 *   len     [B]            int32 verify lengths in [0, gamma] (nullable: gamma)
 *   x       [B][gamma]     int32 draft tokens
 *   ld_lse  [B][gamma]     fp32 logsumexp of the Ld rows, e.g. lse_out of the draft
 *                          (nullable: computed here)
 *   u_acc   [B][gamma]     fp32 acceptance uniforms
 *   u_fin   [B]            fp32 uniform of the residual or bonus draw
 *   n_acc_out [B]          int32 accepted count n_b (-1: a verified draft token was invalid)
 *   y_out   [B][gamma+1]   int32 emitted tokens x_1..x_n, z, then -1
 *   lse_d_out [B][gamma]   fp32 lse of the Ld rows            (nullable; NaN beyond len)
 *   lse_t_out [B][gamma+1] fp32 lse of the target rows        (nullable; NaN beyond len+1)
 * A len outside [0, gamma], or rows t_off[b] .. t_off[b] + len[b] not inside [0, Lt_rows), is
 * a device-data fault: that request gets n = -1 and y all -1 and is otherwise skipped.
 */
size_t dspark_verify_workspace_bytes(int B, int V, int gamma);
int dspark_verify(int B, int V, int gamma,
                  const float* Ld, const float* Lt, int Lt_rows,
                  const int32_t* t_off, const int32_t* len,
                  const int32_t* x, const float* ld_lse, const float* u_acc, const float* u_fin,
                  int32_t* n_acc_out, int32_t* y_out, float* lse_d_out, float* lse_t_out,
                  void* ws, size_t ws_bytes, void* stream);

/*
 * TV soft labels c*_k = 1 - 1/2 ||p_d - p_t||_1 = sum_v min(p_d(v), p_t(v)).
 * [P3] "Confidence-Scheduled Verification" (label of the confidence head); [P1] section
 * "硬件感知与置信度自适应调度机制" (analytic acceptance rate from the total variation distance).
 *
 *   Ld, Lt, Lt_rows, t_off, len   as in dspark_verify (a faulty request gets NaN labels)
 *   lse_d   [B][gamma]   fp32 (nullable: computed)
 *   lse_t   [B][gamma+1] fp32 (nullable: computed)
 *   cstar_out [B][gamma] fp32 c* for k < len[b]; NaN for k >= len[b]
 */
size_t dspark_tv_labels_workspace_bytes(int B, int V, int gamma);
int dspark_tv_labels(int B, int V, int gamma,
                     const float* Ld, const float* Lt, int Lt_rows,
                     const int32_t* t_off, const int32_t* len,
                     const float* lse_d, const float* lse_t, float* cstar_out,
                     void* ws, size_t ws_bytes, void* stream);

/*
 * Verify and TV labels in one call: the same results as dspark_verify followed by
 * dspark_tv_labels on the same rows, bit for bit. Arguments as in dspark_verify, plus
 * cstar_out [B][gamma] fp32 (required) as in dspark_tv_labels. The normalisers of both come
 * from the same row partials, so c* equals what dspark_tv_labels computes from this call's
 * lse_d / lse_t.
 * Rows of at most 64 chunks of 8192 logits (V <= 524288) are read once: a persistent pass
 * keeps each chunk of a row pair in registers until the row's normalisers are known (two
 * launches), or for at most 768 (row, chunk) tasks a single launch that also draws the
 * final token. Longer rows take two passes (normalisers, then acceptance data and TV sums).
 * Every path forms a probability from its chunk's maximum M as exp(x - M) * exp(M - lse).
 * The one-pass forms need every workgroup of the launch resident at once and must not
 * overlap another call on the same workspace.
 */
size_t dspark_verify_tv_workspace_bytes(int B, int V, int gamma);
int dspark_verify_tv(int B, int V, int gamma,
                     const float* Ld, const float* Lt, int Lt_rows,
                     const int32_t* t_off, const int32_t* len, const int32_t* x,
                     const float* ld_lse, const float* u_acc, const float* u_fin,
                     int32_t* n_acc_out, int32_t* y_out, float* lse_d_out, float* lse_t_out,
                     float* cstar_out, void* ws, size_t ws_bytes, void* stream);

/*
 * Verify and TV labels with the draft logits rebuilt from the Markov factors, so that the
 * draft call need not write them (Ld_out NULL). [P3] "Semi-Autoregressive Generation":
 * L_d[b, k] = U[b, k] + W1[x_{k-1}] W2 with x_{-1} = x0; the acceptance test, residual and
 * bonus draws ([P1] section "大模型推理的显存瓶颈与推测解码的演进逻辑") and the labels ([P3]
 * "Confidence-Scheduled Verification") are those of dspark_verify_tv. Only the verified
 * rows (k < len[b]) are rebuilt, with the same bf16 MFMA arithmetic as the slab draft path,
 * whose logits they reproduce bit for bit.
 *
 *   U, W1, W2, w_dtype, x0   the draft call's inputs (bf16 factors only; r <= 256 with
 *                            r % 8 == 0, V % 8 == 0, V <= 163840; U, W1, W2, Lt 16-byte
 *                            aligned)
 *   x       [B][gamma]       int32 draft tokens
 *   ld_lse  [B][gamma]       fp32 draft normalisers from the draft call (required)
 *   Lt, Lt_rows, t_off, len, u_acc, u_fin   as in dspark_verify
 *   n_acc_out, y_out         as in dspark_verify
 *   lse_t_out [B][gamma+1]   fp32 lse of the target rows (nullable; NaN beyond len+1)
 *   cstar_out [B][gamma]     fp32 c* for k < len[b], NaN beyond (nullable)
 * Faulty requests (len or offsets out of range, a token outside [0, V), or an invalid x0
 * with len > 0) get n = -1, y all -1 and NaN labels. Up to rounding order (the final draw
 * sums masses over 16 NT-column tiles instead of 8192-logit chunks) the results equal
 * dspark_verify_tv on the draft's own logits; the acceptance decisions are identical.
 */
size_t dspark_verify_markov_workspace_bytes(int B, int V, int r, int gamma);
int dspark_verify_markov(int B, int V, int r, int gamma,
                         const float* U, const void* W1, const void* W2, int w_dtype,
                         const int32_t* x0, const int32_t* x, const float* ld_lse,
                         const float* Lt, int Lt_rows, const int32_t* t_off, const int32_t* len,
                         const float* u_acc, const float* u_fin,
                         int32_t* n_acc_out, int32_t* y_out, float* lse_t_out, float* cstar_out,
                         void* ws, size_t ws_bytes, void* stream);

/*
 * Hardware-aware prefix scheduler.
 * [P1] section "硬件感知与置信度自适应调度机制" and [P3] "Confidence-Scheduled Verification":
 * per-position temperature calibration c' = 1 / (1 + ((1-c)/c)^(1/T_k)); prefix survival
 * a_{r,j} = prod_{i<=j} c'_{r,i}; all R*gamma candidates ranked by a descending (ties:
 * position ascending, then request ascending); Theta(n) = (R + sum of the top-n a) *
 * SPS(R + n) for n = 0 .. min(R*gamma, Bmax - R); GLOBAL takes the smallest argmax,
 * EARLY_STOP the first n with Theta(n+1) <= Theta(n); len[r] counts request r's candidates
 * among the top n (a prefix of its block).
 *
 *   conf    [R][gamma]  fp32 conditional confidences c in [0, 1]
 *   temp    [gamma]     fp32 per-position temperatures > 0 (nullable: no scaling)
 *   sps     [Bmax+1]    fp32 engine steps/s at B total verify tokens
 *   mode    DSPARK_SCHED_GLOBAL or DSPARK_SCHED_EARLY_STOP
 *   len_out   [R]       int32 verify lengths
 *   t_off_out [R+1]     int32 exclusive scan of len + 1 (nullable)
 *   K_out     [1]       int32 total verify tokens R + n* (nullable)
 *   theta_out [1]       fp32 Theta(n*) (nullable)
 *   a_out   [R][gamma]  fp32 prefix survival (nullable)
 * Up to 64 candidates it runs as one wave; past that as three launches (keys, ranks, the Theta
 * scan and lengths). Each candidate's ranking key keeps the sign, the exponent and 32
 * mantissa bits of its fp64 a (44 bits), then j and r. The workspace holds per candidate the
 * key in row order, the key in ranked order and its rank (R * gamma * 20 bytes).
 */
size_t dspark_schedule_workspace_bytes(int R, int gamma, int Bmax);
int dspark_schedule(int R, int gamma, const float* conf, const float* temp,
                    const float* sps, int Bmax, int mode,
                    int32_t* len_out, int32_t* t_off_out, int32_t* K_out, float* theta_out,
                    float* a_out, void* ws, size_t ws_bytes, void* stream);

/*
 * The draft and the schedule in one call, for callers whose schedule does not depend on this
 * draft (the two-step-lag schedule of [P1] section "硬件感知与置信度自适应调度机制", which
 * takes the scheduler off the step's critical path): the results of dspark_markov_draft
 * followed by dspark_schedule (ring NULL) or dspark_schedule_lagged (ring given; conf is then
 * ignored), bit for bit. gamma is the block length of both; R the schedule's request count.
 * When the draft takes the single-request one-launch form (DSPARK_PATH_RESIDENT) and
 * R * gamma <= 64, the schedule runs in one extra workgroup of the draft's launch, on a
 * compute unit the draft leaves idle (dspark_markov_draft_schedule_fused tells whether a call
 * does); otherwise the schedule is launched after the draft. Argument rules and errors are
 * those of the two calls. Workspace: dspark_markov_draft_schedule_workspace_bytes (the draft's
 * worst-case workspace, then the schedule's).
 */
size_t dspark_markov_draft_schedule_workspace_bytes(int B, int V, int r, int gamma, int R, int Bmax);
int dspark_markov_draft_schedule_fused(int B, int V, int r, int gamma, int w_dtype, const void* W1,
                                       const void* W2, int R);
int dspark_markov_draft_schedule(int B, int V, int r, int gamma,
                                 const float* U, const void* W1, const void* W2, int w_dtype,
                                 const int32_t* x0, const float* u,
                                 int32_t* x_out, float* q_out, float* lse_out, float* Ld_out,
                                 int R, const float* conf, const void* ring, size_t ring_bytes,
                                 const float* temp, const float* sps, int Bmax, int mode,
                                 int32_t* len_out, int32_t* t_off_out, int32_t* K_out,
                                 float* theta_out, float* a_out,
                                 void* ws, size_t ws_bytes, void* stream);

/*
 * Two-step-lag schedule.
 * [P1] section "硬件感知与置信度自适应调度机制" (the asynchronous adaptation): the verify
 * lengths of step t are decided from the confidences predicted at step t - 2, which cannot
 * carry information about the tokens being generated now, so the decision is lossless and
 * its latency hides in the GPU pipeline (no host handshake, compatible with graph replay);
 * [P3] "Confidence-Scheduled Verification": the batch capacity K is predicted from the
 * confidences of two steps earlier.
 *
 * The history is a device buffer (`ring`, dspark_conf_ring_bytes(R, gamma) bytes, 8-byte
 * aligned, owned by the caller): a round counter n and three [R][gamma] fp32 slots.
 *   dspark_conf_ring_init    n = 0 and every slot 1.0 (no history: every position survives)
 *   dspark_conf_ring_push    slot n mod 3 <- conf [R][gamma], then n <- n + 1
 *   dspark_schedule_lagged   dspark_schedule on slot (n - 2) mod 3: the confidences pushed
 *                            two pushes before the next one, i.e. at round t (n = t pushes
 *                            so far, one per earlier round) those of round t - 2, and all
 *                            1.0 for t < 2. Arguments and outputs as dspark_schedule.
 * The slot is chosen on the device from n, so a round (lagged schedule, draft, verify, push)
 * can be captured once and replayed without host synchronisation. Calls on one ring must be
 * ordered (one stream, or events); a push must not overlap a lagged schedule on the same
 * ring. Errors: INVALID_ARG for a NULL or misaligned ring or NULL conf, WORKSPACE when
 * ring_bytes is too small, UNSUPPORTED past the scheduler's R * gamma cap.
 */
size_t dspark_conf_ring_bytes(int R, int gamma);
int dspark_conf_ring_init(int R, int gamma, void* ring, size_t ring_bytes, void* stream);
int dspark_conf_ring_push(int R, int gamma, void* ring, size_t ring_bytes, const float* conf,
                          void* stream);
int dspark_schedule_lagged(int R, int gamma, const void* ring, size_t ring_bytes,
                           const float* temp, const float* sps, int Bmax, int mode,
                           int32_t* len_out, int32_t* t_off_out, int32_t* K_out,
                           float* theta_out, float* a_out, void* ws, size_t ws_bytes,
                           void* stream);

/*
 * Sequential temperature scaling (STS) fit.
 * [P1] section "硬件感知与置信度自适应调度机制": the confidence head's scores are calibrated
 * with one temperature per candidate position, each chosen by a one-dimensional grid search
 * on validation data (the expected calibration error, ECE, is the figure of merit; the
 * scaling keeps the scores' order). [P3] "Confidence-Scheduled Verification": c_k estimates
 * P(position k accepted | its prefix accepted).
 *
 *   conf    [N][gamma] fp32 raw scores of N validation requests
 *   n_acc   [N] int32 accepted counts from dspark_verify (negative: request ignored)
 *   len     [N] int32 verify lengths (nullable -> gamma)
 *   grid    [n_grid] fp32 candidate temperatures (a value <= 0 counts as 1)
 *   bins    number of equal-width ECE bins on [0, 1], 1 <= bins <= 16
 *   objective  DSPARK_STS_NLL: binary negative log-likelihood of the observed outcomes
 *              (probabilities floored at 1e-12); DSPARK_STS_ECE: the ECE itself
 *   T_out   [gamma] fp32 the first grid value minimising the objective
 *   ece_before / ece_after [gamma] fp32 ECE at T = 1 and at T_out
 *   obj_out [gamma][n_grid] fp32 the objective at every grid value (nullable)
 * Outcomes: positions k < n_acc were accepted, position n_acc was rejected when
 * n_acc < len, later positions were not observed. Calibrated score:
 * sigmoid(logit(c) / T) in fp64; the ECE's per-bin sums of (outcome - score) add each term
 * rounded to 2^-30 as an exact integer, so results are bitwise reproducible. Caps: 1 <= N, N * gamma < 2^31, 1 <= gamma <= 64,
 * 1 <= n_grid <= 4096.
 */
enum { DSPARK_STS_NLL = 0, DSPARK_STS_ECE = 1 };
size_t dspark_sts_fit_workspace_bytes(int N, int gamma, int n_grid);
int dspark_sts_fit(int N, int gamma, const float* conf, const int32_t* n_acc, const int32_t* len,
                   const float* grid, int n_grid, int bins, int objective,
                   float* T_out, float* ece_before, float* ece_after, float* obj_out,
                   void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DSPARK_H */
