/*
 * dspark.h — C ABI of the DSpark per-step sampling and verification engine
 * (MI355X / gfx950).
 *
 * Three hot-path calls:
 *   dspark_markov_sample  left-to-right low-rank Markov head: turns the parallel
 *                         draft backbone's block logits into gamma proposals,
 *                         their full proposal distributions q and their
 *                         confidence scores.
 *   dspark_verify         exact verify of the proposals against the target
 *                         distribution p: greedy contiguous-prefix match, or
 *                         min(1, p/q) rejection sampling with a max(p-q, 0)
 *                         residual and a bonus token.
 *   dspark_accept_stats   training-side analytic acceptance: L1 distance,
 *                         accept_rate, tau and the position-weighted
 *                         CE / L1 / BCE loss numerator with report pairs.
 *
 * Sources (the pages this engine is built from):
 *   [FT]  "[2/3] feat(dsv4): implement exact DSpark speculative decoding"
 *         (FreeToken pull request): sections "End-to-end speculative cycle",
 *         "Checkpoint-faithful DSpark architecture", "Exact decoding
 *         semantics" (subsections "Greedy", "Probabilistic").
 *   [MB]  "DSpark Speculative Decoding (Draft Training) Design"
 *         (Megatron-Bridge RFC): sections "Semi-autoregressive draft",
 *         "Training objective", "Acceptance and confidence",
 *         "Loss return contract", "Memory contract for the full-vocabulary
 *         terms".
 *   [PS]  "DeepSeek V4 DSpark NPU Serving Dev Notes" (pypto-serving):
 *         section "Speculative decoding (K=7)", paragraphs "Programs",
 *         "Weights", "Acceptance".
 *
 * Conventions shared by every call
 * --------------------------------
 *  * Every array argument is a caller-owned DEVICE pointer to a dense,
 *    row-major, contiguous array, unless stated otherwise.  The library never
 *    allocates, frees or retains device memory; all scratch lives in the
 *    caller's `workspace` (size from dspark_workspace_size), which must stay
 *    untouched until the work queued on `stream` has finished.
 *  * Every call only enqueues work on `stream` (a hipStream_t; NULL = the
 *    default stream) and returns; it never synchronises.  Calls on different
 *    streams with disjoint workspaces may run concurrently; two calls that
 *    share a workspace must be ordered.  Process-wide state is limited to:
 *    the profiler switch and its pending events, the Markov launch-plan
 *    switch, per device one completion event that chains the library's
 *    one-launch Markov grids and a counter that tags their hand-off words
 *    (dspark_markov_plan), and dspark_verify_noalloc's per-GPU scratch.
 *    Several processes on one GPU share nothing but the device: each has its
 *    own chain and counter, so one-launch Markov grids of two processes are
 *    not ordered against each other; if the other process's kernels keep
 *    compute units busy, a grid's bounded waits give up and flag
 *    DSPARK_FLAG_SYNC_TIMEOUT (no hang).
 *  * Arguments are validated on the host BEFORE anything is enqueued; on any
 *    error nothing is launched and the outputs are left untouched.  Device
 *    memory contents are never read on the host, so value problems found on
 *    the device (NaN logits, a non-positive temperature, zero residual mass)
 *    never abort: they set bits in the per-row `flags` outputs.
 *  * bf16 arrays are passed as uint16_t (IEEE binary32 truncated to its upper
 *    16 bits, i.e. bfloat16).
 *  * Sizes: B = requests, gamma = proposals per block, V = vocabulary,
 *    r = Markov rank, d = draft hidden size.  Row k of the target logits
 *    (k = 0..gamma) is the target distribution after token x_k (x_0 = the
 *    anchor), so target row k-1 verifies proposal x_k and row gamma is the
 *    bonus row ([FT] "End-to-end speculative cycle": one target pass over the
 *    anchor plus the proposals).
 *
 * Random numbers
 * --------------
 *  Every random decision uses Philox4x32-10 (Salmon, Moraes, Dror, Shaw,
 *  "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11) with
 *      key     = (seed & 0xffffffff, seed >> 32)
 *      counter = (i >> 2, (uint32_t)position, request_id, tag)
 *  taking 32-bit output word (i & 3), where i is the token index (or chunk or
 *  sub-chunk index) being scored and `position` is the absolute position of
 *  the token being decided (anchor position + k for proposal / emitted token
 *  k).  Tags:
 *      0 DSPARK_TAG_DRAFT_TOKEN   token-level draft noise
 *      1 DSPARK_TAG_ACCEPT        accept-test uniform (i = 0)
 *      2 DSPARK_TAG_TARGET_TOKEN  token-level residual / bonus noise
 *      3 DSPARK_TAG_DRAFT_CHUNK   chunk-level draft noise
 *      4 DSPARK_TAG_TARGET_CHUNK  chunk-level residual / bonus noise
 *      5 DSPARK_TAG_DRAFT_SUB     sub-chunk-level draft noise
 *      6 DSPARK_TAG_TARGET_SUB    sub-chunk-level residual / bonus noise
 *  Uniforms: Gumbel u = ((w >> 9) + 0.5) * 2^-23 in (0,1); accept
 *  u' = (w >> 8) * 2^-24 in [0,1).  Gumbel noise g = -ln(-ln u).
 *
 *  Sampling from weights w_v >= 0 is a three-level Gumbel-max descent over a
 *  fixed partition of the vocabulary ([FT] "Probabilistic" requires only that
 *  the emitted tokens follow the target distribution exactly):
 *    1. chunk c* = argmax_c (ln W_c + g_c) over chunks of DSPARK_CHUNK = 256
 *       consecutive tokens, W_c the chunk's total weight (chunk tag, i = c);
 *    2. sub-chunk j* = argmax_j (ln W_j + g_j) over the DSPARK_SUB = 16-token
 *       sub-chunks of c* (sub-chunk tag, i = the global index v / 16);
 *    3. token v* = argmax_{v in j*} (ln w_v + g_v) (token tag, i = v).
 *  Ties go to the lowest index.  P(v*) = (W_c/W)(W_j/W_c)(w_v/W_j) = w_v/W
 *  exactly, no prefix sum over the vocabulary is needed, and every level can
 *  be evaluated where its data already is.
 *
 * Sampling policy ([FT] "Probabilistic": p and q are both formed after the
 * request's temperature, top-k and top-p)
 * --------------------------------------------------------------------
 *  Sampled rows: z = logits / T; top-k (if 0 < top_k < V) keeps
 *  {v : z_v >= z_(top_k)} (ties at the boundary kept); top-p (if top_p < 1)
 *  then keeps, within that set renormalised, every v whose probability is at
 *  least that of the m-th most probable kept token, m the smallest count whose
 *  cumulative probability reaches top_p (top_p <= 0 keeps the argmax set).
 *  The distribution is softmax(z) over the kept set.  Greedy rows use the
 *  argmax of the unscaled logits (lowest index on ties) and a one-hot
 *  distribution.
 */
#ifndef DSPARK_H
#define DSPARK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes (return value of every call) ------------------------- */
typedef enum dspark_status {
  DSPARK_OK = 0,
  DSPARK_EINVAL = 1,     /* a required pointer is NULL or a size is <= 0     */
  DSPARK_EDTYPE = 2,     /* unknown logits dtype                             */
  DSPARK_ESHAPE = 3,     /* a size outside the supported range (see below)   */
  DSPARK_EWORKSPACE = 4, /* workspace NULL or smaller than required          */
  DSPARK_EDEVICE = 5     /* a HIP launch or runtime call failed              */
} dspark_status;

/* ---- logits element types ------------------------------------------------ */
enum { DSPARK_BF16 = 1, DSPARK_F32 = 2 };

/* ---- per-row flag bits (uint8_t flags outputs) ---------------------------
 * NEAR_THRESHOLD is the device's own diagnostic: a decision whose fp32 margin
 * was within 1e-6 (relative to max(1, |score|), absolute for accept tests) of
 * flipping.  The others report value problems.  NONFINITE and EMPTY_ROW are
 * properties of a row's data and are reported on every row a request owns
 * (target rows 0..n_draft, every draft row); a request with such a row has
 * unspecified tokens, lengths and q outputs (logits must be finite or -inf;
 * -inf excludes a token).  NEAR_THRESHOLD and RESIDUAL_ZERO are reported on
 * the row where the decision was taken, BAD_POLICY on row 0.               */
enum {
  DSPARK_FLAG_NEAR_THRESHOLD = 1u << 0,
  DSPARK_FLAG_NONFINITE = 1u << 1,      /* the row holds a NaN or +inf      */
  DSPARK_FLAG_RESIDUAL_ZERO = 1u << 2,  /* max(p-q,0) had zero mass: sampled
                                           from p instead                     */
  DSPARK_FLAG_EMPTY_ROW = 1u << 3,      /* no logit above -inf in the row    */
  DSPARK_FLAG_BAD_POLICY = 1u << 4,     /* sampled row with temperature <= 0
                                           or non-finite: treated as greedy  */
  DSPARK_FLAG_SYNC_TIMEOUT = 1u << 5    /* dspark_markov_sample only: a wait
                                           of the one-launch plan for another
                                           workgroup's data gave up (other work
                                           held the device's compute units);
                                           every output of the call is
                                           unspecified                        */
};

/* ---- Philox stream tags --------------------------------------------------- */
enum {
  DSPARK_TAG_DRAFT_TOKEN = 0,
  DSPARK_TAG_ACCEPT = 1,
  DSPARK_TAG_TARGET_TOKEN = 2,
  DSPARK_TAG_DRAFT_CHUNK = 3,
  DSPARK_TAG_TARGET_CHUNK = 4,
  DSPARK_TAG_DRAFT_SUB = 5,
  DSPARK_TAG_TARGET_SUB = 6
};

/* Tokens per level-1 chunk and per level-2 sub-chunk of the sampler. */
#define DSPARK_CHUNK 256
#define DSPARK_SUB 16

/* ---- supported ranges (DSPARK_ESHAPE outside them) ------------------------ */
#define DSPARK_MAX_GAMMA 16
#define DSPARK_MAX_RANK 256      /* r must also be a multiple of 16 */
#define DSPARK_MAX_HIDDEN 65536  /* d                                */
#define DSPARK_MAX_VOCAB (1 << 30)
#define DSPARK_MAX_VERIFY_BATCH 65535  /* B of dspark_verify (one grid row each) */

/* ---- per-request sampling policy: all DEVICE arrays of length B ----------- */
typedef struct dspark_policy {
  const uint8_t* mode;         /* 0 = greedy, 1 = sampled                    */
  const float* temperature;    /* T > 0 for sampled rows (ignored if greedy) */
  const int32_t* top_k;        /* 0 or >= V: off                             */
  const float* top_p;          /* >= 1: off                                  */
  /* top_k and top_p are both given or both NULL; NULL means that no request
   * of the call truncates (the calls then skip every truncation pass, and
   * dspark_markov_sample takes its untruncated one-launch kernel).  One NULL
   * without the other is EINVAL.                                             */
  const uint32_t* request_id;  /* Philox counter word 2                      */
  const int32_t* position;     /* absolute position of the anchor x_0        */
} dspark_policy;

/* ---- workspace sizing ------------------------------------------------------ */
enum {
  DSPARK_OP_MARKOV = 1,
  DSPARK_OP_VERIFY = 2,
  DSPARK_OP_STATS = 3,
  DSPARK_OP_STATS_BACKWARD = 4,
  DSPARK_OP_STATS_MARKOV = 5
};

/* Bytes of device workspace one call of `op` needs at these sizes (for
 * DSPARK_OP_STATS pass N as B; r and d are ignored where they do not apply).
 * Returns 0 for an unknown op or non-positive sizes.  Host-only. */
size_t dspark_workspace_size(int op, int32_t B, int32_t gamma, int32_t V,
                             int32_t r, int32_t d);

/* Human-readable name of a status code (static string).  Host-only. */
const char* dspark_status_string(int status);

/* Library version as major*10000 + minor*100 + patch.  Host-only. */
int dspark_version(void);

/* Diagnostics: per-kernel timing with HIP events (off by default; a
 * process-wide switch).  While enabled, every kernel the library
 * launches is bracketed by two events recorded on its stream.
 * dspark_profile_summary waits for the recorded events, writes one line
 * "<kernel> <launches> <total_ms>" per kernel name into buf (NUL-terminated,
 * truncated to n bytes), forgets the records, and returns 0 or DSPARK_EDEVICE. */
int dspark_profile_enable(int on);
int dspark_profile_summary(char* buf, size_t n);

/* Waits for and destroys every HIP object the library holds: the profiler's
 * pending events and the per-device completion events that order the
 * one-launch Markov grids (created on first use; see dspark_markov_plan).
 * Call it before the HIP runtime is torn down (for example from an exit
 * handler that runs before the process's static destructors); later calls
 * create what they need again.  Not concurrent-safe with calls in flight on
 * other threads.  Returns 0. */
int dspark_release(void);

/* Launch plan of dspark_markov_sample (process-wide, like the profiler
 * switch; read when a call is enqueued).
 *   DSPARK_MARKOV_AUTO (default): one launch for all gamma steps whenever its
 *     grid (one workgroup per 512 tokens of the vocabulary) fits the compute
 *     units the stream may use, resident at once; each workgroup then keeps
 *     its slice of markov_w2 in registers for the whole call, the whole
 *     batch takes each step together, and the steps hand their results to
 *     one another through the workspace (polled, no device-wide barrier;
 *     every hand-off word carries a per-call tag, so the workspace needs no
 *     clearing and a stale word is never read as this call's).  It is an
 *     ordinary launch: the library chains its own such launches on a device
 *     (each waits for the previous one's completion event, whatever the
 *     stream; not inside a stream capture), and residency otherwise relies
 *     on no other kernel holding compute units indefinitely.  Every such
 *     wait is bounded: on expiry the call ends and flags its rows
 *     DSPARK_FLAG_SYNC_TIMEOUT.  Otherwise 2 gamma launches as below.
 *   DSPARK_MARKOV_PER_STEP: 2 gamma launches (one stream kernel over all
 *     chunks and one finalize kernel over all requests per step).
 *   DSPARK_MARKOV_COOPERATIVE: as AUTO, but through cooperative launch (the
 *     runtime guarantees residency, at the price of synchronising its
 *     separate queue with the stream before and after the launch).
 *     Without cooperative launch, as PER_STEP.
 *   DSPARK_MARKOV_REQUEST_GROUPS: as AUTO, but without truncation arrays,
 *     with 33 to 256 requests and at least one compute unit to spare, the
 *     requests are taken in groups of 16 whose steps interleave (a group's
 *     hand-off runs while the other groups stream), with one or two extra
 *     workgroups that only combine the records.  Otherwise as AUTO.
 * Inside a stream capture the plans run as outside it (COOPERATIVE as an
 * ordinary launch).  A graph replays its launch arguments, so a captured
 * one-launch kernel takes its hand-off tag from a counter in the workspace
 * instead of the host (advanced by each replay; tags of captured and of
 * eager calls never coincide).  The chaining of one-launch launches is not
 * recorded in the graph: a replay must not run at the same time as another
 * one-launch Markov call on the same GPU (if it does, the bounded waits end
 * the call with DSPARK_FLAG_SYNC_TIMEOUT rows), and replays of graphs that
 * share a workspace must not overlap.
 * All plans compute identical results.  Returns the previous plan, or -1
 * (leaving it unchanged) for an unknown value. */
enum {
  DSPARK_MARKOV_AUTO = 0,
  DSPARK_MARKOV_PER_STEP = 1,
  DSPARK_MARKOV_COOPERATIVE = 2,
  DSPARK_MARKOV_REQUEST_GROUPS = 3
};
int dspark_markov_plan(int plan);

/* ---------------------------------------------------------------------------
 * dspark_markov_sample
 *
 * [FT] "Checkpoint-faithful DSpark architecture": the lightweight Markov head
 * is sampled left to right, proposal k conditioning on proposal k-1 and the
 * first on the anchor; the full proposal distribution q and the confidence
 * scores are kept.  [MB] "Semi-autoregressive draft": the Markov head is a
 * rank-256 token-conditioned additive logit bias, run serially at inference;
 * the confidence head is c_k = sigmoid(w^T [h_k ; embed(x_{k-1})]).
 * [PS] "Weights": markov_w1 / markov_w2, confidence head in FP32.
 *
 * For k = 1..gamma, in order (x_0 = anchor[b]):
 *   y_k   = backbone_logits[b, k-1, :] + markov_w1[x_{k-1}, :] . markov_w2^T
 *           (bias_v = sum_i markov_w1[x_{k-1}, i] * markov_w2[v, i])
 *   q_k   = policy(y_k); x_k ~ q_k (three-level Gumbel-max, draft tags) for a
 *           sampled row, x_k = argmax y_k for a greedy row
 *   c_k   = sigmoid(sum_i conf_w[i] h[b,k-1,i]
 *                   + sum_i conf_w[d+i] embed[x_{k-1}, i])
 *
 * Inputs
 *   backbone_logits  [B, gamma, V]  logits_dtype; row k-1 = draft position k
 *   anchor           [B] int32 in [0, V)
 *   markov_w1        [V, r] bf16: row x is the rank-r code of token x (A)
 *   markov_w2        [V, r] bf16: row v holds the r weights producing logit v
 *                    (the [out, in] Linear layout of the rank-r -> V map)
 *   hidden           [B, gamma, d] bf16: draft hidden state h_k at row k-1
 *   embed            [V, d] bf16: the shared (target) token embedding
 *   conf_w           [2d] fp32: confidence weight over [h_k ; embed(x_{k-1})]
 *   policy, seed     as above
 * Outputs
 *   draft_tokens     [B, gamma] int32: x_1..x_gamma
 *   q_logits         [B, gamma, V] fp32: z = y / T for SAMPLED rows, so that
 *                    q_v = (z_v >= q_thr) ? exp(z_v - q_lse) : 0.  Rows of
 *                    greedy requests are not written (q is one-hot at x_k).
 *   q_lse            [B, gamma] fp32: log-sum-exp of z over the kept set
 *                    (0 for greedy rows)
 *   q_thr            [B, gamma] fp32: smallest kept z when top-k / top-p is
 *                    active, -inf otherwise (0 for greedy rows)
 *   q_tok            [B, gamma] fp32: q_k(x_k) (1 for greedy rows)
 *   confidence       [B, gamma] fp32: c_k
 *   flags            [B, gamma] uint8: DSPARK_FLAG_* per draft row
 * Errors: EINVAL (NULL pointer, size <= 0), EDTYPE, ESHAPE (gamma >
 * DSPARK_MAX_GAMMA, r > DSPARK_MAX_RANK or r % 16 != 0, d > DSPARK_MAX_HIDDEN,
 * V > DSPARK_MAX_VOCAB), EWORKSPACE, EDEVICE.  anchor values outside [0, V)
 * are clamped into range on the device.
 * ------------------------------------------------------------------------- */
dspark_status dspark_markov_sample(
    const void* backbone_logits, int logits_dtype, const int32_t* anchor,
    const uint16_t* markov_w1, const uint16_t* markov_w2,
    const uint16_t* hidden, const uint16_t* embed, const float* conf_w,
    dspark_policy policy, uint64_t seed, int32_t B, int32_t gamma, int32_t V,
    int32_t r, int32_t d, int32_t* draft_tokens, float* q_logits,
    float* q_lse, float* q_thr, float* q_tok, float* confidence,
    uint8_t* flags, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * dspark_verify
 *
 * [FT] "Exact decoding semantics".  Greedy: accept the contiguous prefix of
 * proposals equal to the target argmax, stop at the first disagreement and
 * emit the target token there; a later accidental match is never accepted.
 * Probabilistic: accept x_k with probability min(1, p(x_k)/q(x_k)); at the
 * first rejection sample from normalised max(p - q, 0); if every proposal
 * survives, sample a bonus token from the target's next-position
 * distribution.  [PS] "Acceptance": 1..gamma+1 tokens per step.
 *
 * Per request b with n_d = n_draft[b] (gamma if n_draft is NULL; values are
 * clamped into [0, gamma]):
 *   greedy : t_k = argmax target[b,k,:] (lowest index); n = first k in
 *            [1, n_d] with x_k != t_{k-1}, minus 1 (n_d if none);
 *            out = (x_1..x_n, t_n)
 *   sampled: p_k = policy(target[b,k,:]); accept x_k iff
 *            u'_k < p_{k-1}(x_k) / q_k(x_k) (accept iff p > 0 when q = 0);
 *            first reject j: out = (x_1..x_{j-1}, r), r ~ max(p_{j-1} - q_j, 0)
 *            (target tags, position anchor+j; zero mass: r ~ p_{j-1} and
 *            DSPARK_FLAG_RESIDUAL_ZERO); all accepted: out = (x_1..x_{n_d}, r),
 *            r ~ p_{n_d} (target tags, position anchor+n_d+1).
 *
 * Inputs
 *   target_logits  [B, gamma+1, V] logits_dtype
 *   draft_tokens   [B, gamma] int32
 *   q_logits, q_lse, q_thr, q_tok  as written by dspark_markov_sample; the
 *                  first three may be NULL only if every request is greedy
 *                  (they are then never read); q_tok may be NULL likewise.
 *   n_draft        [B] int32 or NULL
 *   policy, seed   the same policy/seed as the Markov call
 * Outputs
 *   accept_len     [B] int32: accepted proposals n in [0, n_d]
 *   out_tokens     [B, gamma+1] int32: the n+1 emitted tokens, then -1
 *   flags          [B, gamma+1] uint8: bits per target row
 * Errors: as dspark_markov_sample (gamma range, V range), and ESHAPE for
 * B > DSPARK_MAX_VERIFY_BATCH.
 * ------------------------------------------------------------------------- */
dspark_status dspark_verify(
    const void* target_logits, int logits_dtype, const int32_t* draft_tokens,
    const float* q_logits, const float* q_lse, const float* q_thr,
    const float* q_tok, const int32_t* n_draft, dspark_policy policy,
    uint64_t seed, int32_t B, int32_t gamma, int32_t V, int32_t* accept_len,
    int32_t* out_tokens, uint8_t* flags, void* workspace,
    size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * dspark_verify_noalloc
 *
 * For callers that cannot allocate device memory or pass a workspace (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): dspark_verify with the same arguments, semantics, outputs and
 * errors, minus workspace and workspace_bytes.  Its scratch is a
 * DSPARK_NOALLOC_SCRATCH_BYTES array of device memory owned by the library,
 * one copy per GPU, held until the process ends; the call itself allocates
 * nothing.  Every call on a GPU shares that GPU's copy: calls that overlap on
 * one GPU (other streams, other threads) race, so order them.  The scratch
 * keeps the last call's contents; the call clears what must start at zero.
 * Errors: as dspark_verify, and EWORKSPACE when the call needs more than
 * DSPARK_NOALLOC_SCRATCH_BYTES (dspark_workspace_size(DSPARK_OP_VERIFY, ...)
 * bounds the need: 1.5 MiB at B = 64, gamma = 5, V = 129280).
 * ------------------------------------------------------------------------- */
#define DSPARK_NOALLOC_SCRATCH_BYTES (32u << 20)

dspark_status dspark_verify_noalloc(
    const void* target_logits, int logits_dtype, const int32_t* draft_tokens,
    const float* q_logits, const float* q_lse, const float* q_thr,
    const float* q_tok, const int32_t* n_draft, dspark_policy policy,
    uint64_t seed, int32_t B, int32_t gamma, int32_t V, int32_t* accept_len,
    int32_t* out_tokens, uint8_t* flags, void* stream);

/* ---------------------------------------------------------------------------
 * dspark_accept_stats
 *
 * [MB] "Training objective", "Acceptance and confidence", "Loss return
 * contract".  For every block b in [0, N) and position k = 1..gamma (row k-1),
 * with P = softmax(draft[b,k-1,:]) and T = softmax(target[b,k-1,:]):
 *   l1   = sum_v |P_v - T_v|                (raw L1; the 1/2 is only in a)
 *   a    = clamp(1 - 0.5 * l1, 0, 1)        (accept_rate)
 *   ce   = logsumexp(draft row) - draft[b,k-1,teacher[b,k-1]]
 *   bce  = max(c,0) - c*a + log1p(exp(-|c|)),  c = conf_logits[b,k-1]
 *   tau_b = 1 + sum_k prod_{j<=k} a_{b,j}
 * and with w_k = exp(-k/gamma) and mask_b = block_mask[b] != 0:
 *   sums[0]  numerator  = sum_b mask_b sum_k w_k (w_ce ce + w_l1 l1 + w_conf bce)
 *   sums[1]  num_tokens = gamma * sum_b mask_b
 *   report pairs [sum, count] over masked positions (blocks for tau):
 *   sums[2..3] l1, sums[4..5] accept_rate, sums[6..7] tau, sums[8..9] ce,
 *   sums[10..11] bce.
 * The numerator is never normalised here: callers divide once by the
 * globally reduced num_tokens, and form logged ratios as sum/count.
 *
 * Inputs : draft_logits, target_logits [N, gamma, V] logits_dtype;
 *          teacher [N, gamma] int32 (clamped into [0, V)); conf_logits
 *          [N, gamma] fp32; block_mask [N] uint8 or NULL (all ones);
 *          w_ce, w_l1, w_conf host scalars (0.1, 0.9, 1.0 in the pages).
 * Outputs: l1, accept_rate, ce, bce [N, gamma] fp32 (every block, masked or
 *          not); tau [N] fp32; sums [12] fp32.
 * Errors : EINVAL, EDTYPE, ESHAPE (gamma, V ranges), EWORKSPACE, EDEVICE.
 * ------------------------------------------------------------------------- */
dspark_status dspark_accept_stats(
    const void* draft_logits, const void* target_logits, int logits_dtype,
    const int32_t* teacher, const float* conf_logits,
    const uint8_t* block_mask, int32_t N, int32_t gamma, int32_t V,
    float w_ce, float w_l1, float w_conf, float* l1, float* accept_rate,
    float* ce, float* bce, float* tau, float* sums, void* workspace,
    size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * dspark_accept_stats_markov
 *
 * [MB] "Semi-autoregressive draft" (the Markov head adds a low-rank,
 * token-conditioned bias to the parallel logits; at training time it is
 * teacher-forced with the previous block tokens) and the statistics of
 * dspark_accept_stats.  The draft row of block b at position k is formed on
 * the device, never stored:
 *   draft[b,k-1,:] = backbone[b,k-1,:] + W1[x_{k-1}] . W2^T
 *   x_0 = anchor[b],  x_{k-1} = teacher[b,k-2] for k >= 2  (clamped to [0,V))
 * and l1, accept_rate, ce, bce, tau and sums are those of dspark_accept_stats
 * on these rows and target_logits.  The bias is an MFMA contraction of
 * 2 N gamma V r flops per look at the rows (two looks).
 *
 * Inputs
 *   backbone_logits [N, gamma, V] logits_dtype (the parallel draft logits)
 *   target_logits   [N, gamma, V] logits_dtype
 *   anchor          [N] int32
 *   markov_w1, markov_w2  [V, r] bf16 (16-byte aligned), r as in
 *                   dspark_markov_sample
 *   teacher, conf_logits, block_mask, N, gamma, V, w_ce, w_l1, w_conf
 *                   as dspark_accept_stats
 * Outputs: as dspark_accept_stats.
 * Workspace: dspark_workspace_size(DSPARK_OP_STATS_MARKOV, N, gamma, V, r, 0).
 * Errors: as dspark_accept_stats, plus EINVAL (NULL anchor or factors,
 * r <= 0, misaligned factors) and ESHAPE (r > DSPARK_MAX_RANK or r % 16 != 0).
 * ------------------------------------------------------------------------- */
dspark_status dspark_accept_stats_markov(
    const void* backbone_logits, const void* target_logits, int logits_dtype,
    const int32_t* anchor, const uint16_t* markov_w1, const uint16_t* markov_w2,
    int32_t r, const int32_t* teacher, const float* conf_logits,
    const uint8_t* block_mask, int32_t N, int32_t gamma, int32_t V,
    float w_ce, float w_l1, float w_conf, float* l1, float* accept_rate,
    float* ce, float* bce, float* tau, float* sums, void* workspace,
    size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * dspark_accept_stats_backward
 *
 * [MB] "Training objective" (the draft is trained by w_ce CE + w_l1 raw L1;
 * the BCE term trains the confidence head against the acceptance label; the
 * target distribution is detached) and "Memory contract for the
 * full-vocabulary terms" (the row chunks are recomputed in the backward).
 * The gradient of scale * sums[0] of dspark_accept_stats (same inputs and
 * weights), with the label a held fixed in the BCE:
 *   grad_draft[b,k-1,v] = scale m_b w_k [ w_ce (P_v - [v == teacher])
 *                                        + w_l1 P_v (s_v - sum_u s_u P_u) ]
 *   grad_conf[b,k-1]    = scale m_b w_k w_conf (sigmoid(c) - a)
 * with P, T, a, w_k, m_b as in dspark_accept_stats, s_u = sign(P_u - T_u)
 * and sign(0) = 0 (the subgradient of |x| that vanishes at 0).  No gradient
 * is produced for the target rows.  Each row pair is read three times
 * (normalisers; L1 and S; the gradient row), the gradient written once.
 *
 * Inputs
 *   draft_logits, target_logits, teacher, conf_logits, block_mask, N, gamma,
 *   V, w_ce, w_l1, w_conf   as dspark_accept_stats
 *   grad_scale  device float32 scalar or NULL (1): the upstream gradient of
 *               the numerator (for example 1 / num_tokens of the loss)
 * Outputs
 *   grad_draft  [N, gamma, V] in logits_dtype (bf16: rounded to nearest even)
 *   grad_conf   [N, gamma] float32
 * Workspace: dspark_workspace_size(DSPARK_OP_STATS_BACKWARD, N, gamma, V, 0, 0)
 * (0 is valid when it returns 0).  Errors: as dspark_accept_stats.  N = 0 is
 * a no-op.
 * ------------------------------------------------------------------------- */
dspark_status dspark_accept_stats_backward(
    const void* draft_logits, const void* target_logits, int logits_dtype,
    const int32_t* teacher, const float* conf_logits,
    const uint8_t* block_mask, int32_t N, int32_t gamma, int32_t V,
    float w_ce, float w_l1, float w_conf, const float* grad_scale,
    void* grad_draft, float* grad_conf, void* workspace,
    size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * dspark_select_width
 *
 * [FT] scope notes and the author's reply on hardware-aware width: a measured
 * choice over 0..gamma proposals that declines or shortens speculation when
 * the draft plus verify cost D + V(k) does not pay.  [MB] "Overview": the
 * confidence head predicts per-position acceptance so that the server can
 * schedule its verify budget.  Per request b, with c_j = confidence[b, j-1]
 * clamped to [0, 1] (NaN -> 0) read as the probability that proposal j is
 * accepted once 1..j-1 were:
 *   E(w)       = 1 + sum_{k<=w} prod_{j<=k} c_j   (expected tokens emitted when
 *                the first w proposals are verified; E(gamma) is tau of
 *                dspark_accept_stats with c for a)
 *   n_draft[b] = the w in [0, gamma] with the largest E(w) / (D + V(w)); the
 *                smaller w on ties; a w whose D + V(w) is not a finite
 *                positive number is skipped (none left: 0)
 * evaluated in binary64 in the order p_k = p_{k-1} c_k, E_k = E_{k-1} + p_k,
 * E / (D + V(w)), every operation rounded separately (no fused multiply-add),
 * so the choice is exact and reproducible.  n_draft feeds dspark_verify.
 *
 * Inputs
 *   confidence [B, gamma] float32 (as written by dspark_markov_sample)
 *   cost       [gamma + 2] float32, device memory: {D, V(0), ..., V(gamma)}
 *              in one time unit of the caller's choice
 * Outputs
 *   n_draft    [B] int32
 *   expected   [B] float32 or NULL: E(n_draft[b])
 * No workspace.  Errors: EINVAL (NULL confidence, cost or n_draft; B < 0;
 * gamma <= 0), ESHAPE (gamma > DSPARK_MAX_GAMMA), EDEVICE.  B = 0 is a no-op
 * (cost must still be given).
 * ------------------------------------------------------------------------- */
dspark_status dspark_select_width(const float* confidence, const float* cost,
                                  int32_t B, int32_t gamma, int32_t* n_draft,
                                  float* expected, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DSPARK_H */
