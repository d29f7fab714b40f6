/*
 * spec_verify.h -- C ABI of the MI355X (gfx950) lossless speculative-sampling
 * verification library (libspecverify.so).
 *
 * What the library computes (pages as published):
 *  - Token-level verification: "Speculative Decoding: The Same Distribution,
 *    Twice as Fast" (derpx06.online), sections 3 "The loop" and 4 "The rule
 *    that makes it exact"; "How much does a token cost" (blog.luminal.com),
 *    section "On Speculative Sampling".
 *  - Block verification: blog.luminal.com, section "Block verification".
 *  - Confidence prefix scheduler: "DeepSeek Boosts Inference Speed by 85%"
 *    (kongchang.com), section "The Third Ace"; "DeepSeek DSpark 详解"
 *    (zskr.cn), section 04.
 *  - Markov-head draft sampler: kongchang.com, section "The First Ace";
 *    zskr.cn, section 03.
 *
 * Conventions for every call:
 *  - Tensor pointers are DEVICE pointers on the context's device, row-major
 *    and contiguous, owned by the caller.  Logit rows must start on a 2-byte
 *    (bf16) or 4-byte (fp32) boundary; 16-byte alignment is faster.
 *  - Layouts: p (target logits) [B, gamma+1, V]; q (draft logits) [B, gamma, V];
 *    draft tokens [B, gamma] int32.  q row i pairs with p row i (i = 1..gamma);
 *    p row gamma+1 is the bonus row.  V is innermost.
 *  - A row's distribution is softmax(logit / temperature).
 *  - Uniforms: Philox4x32-10 (Salmon et al., SC'11) with key = seed and
 *    counter = (request, position | tag << 16, offset lo32, offset hi32),
 *    u = (word0 >> 8) * 2^-24.  Tags: 0 = acceptance test u_i (block:
 *    threshold eta_i), 1 = correction / bonus draw, 2 = Markov draft draw.
 *    Advance `offset` every round so rounds never reuse counters.
 *  - Every *_run call is stream-ordered: it validates its arguments on the
 *    host (synchronously), enqueues kernels on `stream` and returns.  It never
 *    allocates or synchronises.  Argument errors return a status and leave
 *    outputs untouched; the message is in spec_verify_last_error().
 *  - Data errors found on the device (token id outside [0, V), a needed row
 *    that is all -inf or holds NaN/+inf, a verify_len outside [0, gamma]) set
 *    accepted_len[b] = -1 and out_tokens[b, :] = -1 for that request and OR a
 *    flag into the context's device error word (spec_verify_device_status).
 *  - A context is not thread-safe and keeps per-call scratch: use one context
 *    per concurrently running stream.  Calls on one context must be ordered
 *    (same stream, or explicitly synchronised).
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct sv_ctx sv_ctx;

typedef enum {
    SV_OK = 0,
    SV_ERR_INVALID = 1,      /* bad argument (null pointer, size out of range, ...) */
    SV_ERR_UNSUPPORTED = 2,  /* valid but unsupported combination (dtype, size)     */
    SV_ERR_HIP = 3,          /* a HIP runtime call or kernel launch failed          */
    SV_ERR_NOMEM = 4         /* device allocation failed (create only)              */
} sv_status;

typedef enum { SV_F32 = 0, SV_BF16 = 1 } sv_dtype;

/* Device error word / per-request flag bits. */
#define SV_FLAG_BAD_TOKEN      1u  /* draft or anchor token outside [0, V)              */
#define SV_FLAG_BAD_ROW        2u  /* a needed row is all -inf or holds NaN / +inf      */
#define SV_FLAG_RESID_ZERO     4u  /* residual mass rounded to 0: the p row was used    */
#define SV_FLAG_BAD_VERIFY_LEN 8u  /* verify_len[b] outside [0, gamma]                  */

/* Optional diagnostics: a HOST struct of nullable DEVICE pointers (fp32
 * unless noted).  Entries of positions a request did not evaluate are NaN. */
typedef struct {
    float *lse_p;        /* [B, gamma+1] natural log-sum-exp of p rows (after 1/T)   */
    float *lse_q;        /* [B, gamma]   natural log-sum-exp of q rows                */
    float *ratio;        /* [B, gamma]   min(1, p(x_i) / q(x_i))                      */
    float *w;            /* [B, gamma]   block: running capped ratio w_i              */
    float *h;            /* [B, gamma]   block: acceptance threshold h_i              */
    float *resid_mass;   /* [B]          mass Z of the correction / bonus weights     */
    uint32_t *flags;     /* [B]          SV_FLAG_* bits of the request                */
    float *uniform;      /* [B, gamma+1] the uniforms the decisions used: column i-1  */
                         /* u_i (block: eta_i) for i <= L, column gamma the          */
                         /* correction / bonus draw's (not written by tree calls)    */
} sv_diag;

/* Creates a context on `device` for calls with B <= max_batch,
 * gamma <= max_gamma (<= 64), vocabulary `vocab` (1 <= V < 2^31) and, for
 * markov_draft_run, rank `max_rank` (a multiple of 32, or 0 if unused).
 * Allocates the context's device workspace (the only allocation the library
 * makes).  On failure *out is NULL and the status says why. */
sv_status spec_verify_create(sv_ctx **out, int device, int max_batch, int max_gamma,
                             int64_t vocab, int max_rank);

/* Frees the context and its workspace.  The caller must have synchronised
 * every stream that used it.  NULL is accepted. */
void spec_verify_destroy(sv_ctx *ctx);

/* Message of the last failed call on this host thread ("" if none). */
const char *spec_verify_last_error(void);

/* Synchronises `stream`, returns the OR of SV_FLAG_* raised by the device
 * since the last call in *flags, and clears the word. */
sv_status spec_verify_device_status(sv_ctx *ctx, hipStream_t stream, uint32_t *flags);

/* Token-level verification.
 * For each request b, with L = verify_len[b] (gamma when verify_len is NULL):
 * accept x_i with probability min(1, p_i(x_i) / q_i(x_i)), walking i = 1..L
 * and stopping at the first rejection (tau = number accepted); on a rejection
 * draw the correction from max(p_{tau+1} - q_{tau+1}, 0) / Z; if all L pass,
 * draw the bonus token from p_{L+1}.  Draws are inverse-CDF over token ids in
 * ascending order (the smallest id whose cumulative weight exceeds u * Z).
 *   p_logits      [B, gamma+1, V], dtype p_dtype (SV_BF16 or SV_F32)
 *   q_logits      [B, gamma, V],   dtype q_dtype (ignored when gamma == 0)
 *   draft_tokens  [B, gamma] int32
 *   verify_len    [B] int32 or NULL
 *   uniforms      [B, gamma+1] fp32 or NULL: replaces the Philox draws
 *                 (column i-1 = u_i, column gamma = correction/bonus draw)
 *   accepted_len  [B] int32 out: tau_b, or -1 on a data error
 *   out_tokens    [B, gamma+1] int32 out: x_1..x_tau, y, then -1
 *   diag          NULL or diagnostics (see sv_diag)
 * Requires 0 < B <= max_batch, 0 <= gamma <= max_gamma, V == the context's
 * vocab, 0 < temperature < inf. */
sv_status spec_verify_run(sv_ctx *ctx, hipStream_t stream,
                          const void *p_logits, sv_dtype p_dtype,
                          const void *q_logits, sv_dtype q_dtype,
                          const int32_t *draft_tokens, const int32_t *verify_len,
                          int B, int gamma, int64_t V, float temperature,
                          uint64_t seed, uint64_t offset, const float *uniforms,
                          int32_t *accepted_len, int32_t *out_tokens, const sv_diag *diag);

/* Token-level verification without a context and without allocating: for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  Same arguments,
 * kernels and results as spec_verify_run, on the CURRENT HIP device; the
 * call's scratch (row-chunk statistics, request state, correction-weight
 * segment sums) lives in a file-scope device array of the library, 8 MiB
 * per GPU, held until the process ends, found with hipGetSymbolAddress on
 * the first call on each device.  A call needs 256-byte-aligned space for
 * B (2 gamma + 1) ceil(V / chunk) float2 (chunk about 16K tokens), B
 * ceil(V / 2048) floats and B 32-byte request states (about 0.3 MiB at
 * B = 256, gamma = 7, V = 129,280); a larger call returns
 * SV_ERR_UNSUPPORTED and launches nothing.  Every call on a GPU shares that
 * GPU's array: calls that overlap on one GPU (several streams, several host
 * threads) race and must be serialised by the caller.  There is no device
 * error word to read: data errors show per request (accepted_len = -1,
 * diag->flags).  No hipMalloc, hipFree or hipMemset is issued. */
sv_status spec_verify_run_noalloc(hipStream_t stream,
                                  const void *p_logits, sv_dtype p_dtype,
                                  const void *q_logits, sv_dtype q_dtype,
                                  const int32_t *draft_tokens, const int32_t *verify_len,
                                  int B, int gamma, int64_t V, float temperature,
                                  uint64_t seed, uint64_t offset, const float *uniforms,
                                  int32_t *accepted_len, int32_t *out_tokens, const sv_diag *diag);

/* Hardware-aware prefix scheduler.  Survival S_{b,i} = prod_{j<=i} conf_{b,j}
 * (binary64); candidates are ranked by (S descending, b ascending, i
 * ascending) and admitted one by one while E * SPS(rows) strictly rises, with
 * SPS(n) = sps_a / (1 + n / sps_k), E starting at B and rows at B (every
 * request verifies its correction/bonus row); the first candidate that does
 * not raise it stops admission.
 *   conf          [B, gamma] fp32, each in [0, 1] (values outside are clamped)
 *   verify_len    [B] int32 out
 *   expected      [1] fp64 out or NULL: E of the chosen allocation
 * Requires B * gamma <= 8192 (one workgroup sorts every candidate in LDS). */
sv_status spec_schedule_run(sv_ctx *ctx, hipStream_t stream, const float *conf,
                            int B, int gamma, float sps_a, float sps_k,
                            int32_t *verify_len, double *expected);

/* The prefix scheduler on temperature-scaled confidences ("DeepSeek Boosts
 * Inference Speed by 85%", section "The Second Ace"; "DeepSeek DSpark 详解",
 * section 04): position i of every request has its own temperature T_i, and
 * the confidence of candidate (b, i) is 1 / (1 + exp(-conf_logits[b,i] / T_i))
 * (binary64; NaN is taken as 0); ranking and admission then as
 * spec_schedule_run.
 *   conf_logits   [B, gamma] fp32 device: the confidence head's log-odds
 *   temperatures  [gamma] fp32 HOST pointer, each finite and > 0; read
 *                 during the call, which copies them into the launch
 * The scheduler reads only confidences, never draft tokens or uniforms, so
 * it may run ahead of verification: a serving loop can call it on a second
 * stream (with a second context, a context being single-stream) on the
 * estimates of an earlier step and hand verify_len over with an event, which
 * takes it off the verification stream's critical path (the two-step-delayed
 * schedule of "DeepSeek Boosts Inference Speed by 85%", section "The Third
 * Ace", and "DSpark: DeepSeek's bet on speed that doesn't betray quality",
 * section "Verifying only what matters").  Make that second stream
 * non-blocking (hipStreamNonBlocking): a blocking stream also orders itself
 * against the null stream, which serialises the handover. */
sv_status spec_schedule_sts_run(sv_ctx *ctx, hipStream_t stream, const float *conf_logits,
                                const float *temperatures, int B, int gamma, float sps_a, float sps_k,
                                int32_t *verify_len, double *expected);

/* Block verification: keeps the longest passing prefix.  With running ratio
 * w_0 = 1, w_i = min(1, w_{i-1} p_i(x_i) / q_i(x_i)), residual masses
 * m_i = sum_v max(w_i p_{i+1}(v) - q_{i+1}(v), 0), thresholds
 * h_i = m_i / (m_i + 1 - w_i) for i < L (1 when 0/0) and h_L = w_L,
 * tau = the largest i in 1..L with eta_i < h_i (else 0); the correction is
 * drawn from max(w_tau p_{tau+1} - q_{tau+1}, 0) or, for tau = L, the bonus
 * from p_{L+1}.  With L = 1 it takes token verification's decisions.
 * If `conf` is non-NULL the scheduler runs first on the same stream and its
 * verify_len (written to verify_len_out when non-NULL) drives the call;
 * otherwise `verify_len` (or gamma) does.  Other arguments as
 * spec_verify_run. */
sv_status spec_blockverify_run(sv_ctx *ctx, hipStream_t stream,
                               const void *p_logits, sv_dtype p_dtype,
                               const void *q_logits, sv_dtype q_dtype,
                               const int32_t *draft_tokens, const int32_t *verify_len,
                               const float *conf, float sps_a, float sps_k,
                               int32_t *verify_len_out,
                               int B, int gamma, int64_t V, float temperature,
                               uint64_t seed, uint64_t offset, const float *uniforms,
                               int32_t *accepted_len, int32_t *out_tokens, const sv_diag *diag);

/* Tree verification ("Speculative Decoding: The Same Distribution, Twice as
 * Fast", section 7: several alternative continuations arranged as a tree,
 * checked in one pass).  The page gives no rule; this is recursive rejection,
 * lossless when the children of each node were drawn independently from the
 * draft distribution at that node.  From the root, at each node in turn:
 * every child x, in node order, is accepted with probability
 * min(1, r(x) / q(x)) for the current residual r (p at the node, and after
 * each rejection max(r - q, 0) normalised); an accepted child is emitted and
 * the walk continues there; if every child is rejected the final token is
 * drawn from r, and at a leaf the bonus token from p (inverse CDF in token
 * order).  The first child's test is spec_verify_run's, so a chain (node m's
 * parent m - 1) gives spec_verify_run's result with gamma = N.
 *   parents       HOST [N]: parent of node m (1..N) at index m-1, in
 *                 [0, m-1]; node 0 is the root; one topology for the batch
 *   p_logits      [B, N+1, V]: row n = target logits after node n
 *   q_logits      [B, NQ, V]: draft logits at each node that has children,
 *                 in node order (NQ = the number of such nodes)
 *   tokens        [B, N] int32: token of node m at column m-1
 *   uniforms      [B, N+1] fp32 or NULL: column m-1 replaces node m's test
 *                 uniform (Philox (b, m, tag 0)), column N the final draw's
 *                 ((b, 0, tag 1))
 *   accepted_len  [B] int32 out: depth of the accepted path, -1 on a data error
 *   out_tokens    [B, D+1] int32 out (D = the tree's depth): the accepted
 *                 path's tokens, the drawn token, then -1
 *   accepted_nodes [B, D] int32 out or NULL: the accepted nodes, then -1
 *   diag          NULL or lse_p [B, N+1], lse_q [B, NQ], ratio [B, N]
 *                 (min(1, r(x)/q(x)) of each tested node, NaN otherwise),
 *                 resid_mass [B], flags [B]
 * Requires N <= max_gamma, V == the context's vocab, V <= 8.4M; every token
 * in [0, V) and every row finite (else accepted_len = -1 and a flag). */
sv_status tree_verify_run(sv_ctx *ctx, hipStream_t stream,
                          const void *p_logits, sv_dtype p_dtype,
                          const void *q_logits, sv_dtype q_dtype,
                          const int32_t *tokens, const int32_t *parents, int N,
                          int B, int64_t V, float temperature, uint64_t seed, uint64_t offset,
                          const float *uniforms, int32_t *accepted_len, int32_t *out_tokens,
                          int32_t *accepted_nodes, const sv_diag *diag);

/* Markov-head draft sampler.  For k = 1..gamma, strictly left to right:
 * z_k[n] = base_k[n] + sum_r U[x_{k-1}, r] W[r, n] (bf16 inputs, fp32
 * accumulation), x_k = inverse-CDF draw from softmax(z_k / temperature) with
 * uniform tag 2 at position k.  x_0 is the anchor token.
 *   base_logits   [B, gamma, V] bf16
 *   U             [V, R] bf16: row x is the transition embedding of token x
 *   Wt            [V, R] bf16: W stored vocabulary-major (Wt[n, r] = W[r, n]),
 *                 the way a linear layer from R to V stores its weight
 *   R             == the context's max_rank
 *   x0            [B] int32 anchor tokens
 *   uniforms      [B, gamma] fp32 or NULL (replaces the Philox draws)
 *   draft_tokens  [B, gamma] int32 out
 *   q_logits      [B, gamma, V] fp32 out or NULL: z_k before 1/temperature
 *   lse_q         [B, gamma] fp32 out or NULL: log-sum-exp of z_k / T
 * Requires R == the context's max_rank and V <= 262,144 (SV_ERR_UNSUPPORTED
 * beyond); U and Wt must be 16-byte aligned. */
sv_status markov_draft_run(sv_ctx *ctx, hipStream_t stream,
                           const void *base_logits, const void *U, const void *Wt, int R,
                           const int32_t *x0, int B, int gamma, int64_t V, float temperature,
                           uint64_t seed, uint64_t offset, const float *uniforms,
                           int32_t *draft_tokens, float *q_logits, float *lse_q);

/* Markov-head draft followed by token-level verification of that draft,
 * without materialising the draft logits.  The draft is markov_draft_run's
 * (seed draft_seed, offset; Markov head: "DeepSeek Boosts Inference Speed by
 * 85%" (kongchang.com), section "The First Ace"); the verification is
 * spec_verify_run's token rule (seed verify_seed, same offset; "Speculative
 * Decoding: The Same Distribution, Twice as Fast", section 4) with q the
 * softmax of the draft logits at the same temperature.  The sampler supplies
 * each draft row's normaliser and the drafted tokens' logits; the one draft
 * row per request that the residual max(p - q, 0) needs (position tau + 1) is
 * rebuilt after the acceptance scan with the sampler's own arithmetic, so it
 * equals the row the token was drawn from, and weighed as it is built: the
 * correction / bonus weights are summed per 64-token tile and the token is
 * drawn from those sums and the chosen tile's weights (rebuilt again the same
 * way), so no draft row is ever stored.  Decisions equal those of
 * markov_draft_run then spec_verify_run up to the fp32 rounding of the draft
 * normalisers (the two paths sum them in different orders).
 *   base_logits [B, gamma, V] bf16; U, Wt [V, R] bf16 (16-byte aligned);
 *   x0 [B] int32 anchors; p_logits [B, gamma+1, V] (bf16 or fp32)
 *   draft_tokens [B, gamma] int32 out; accepted_len [B], out_tokens
 *   [B, gamma+1] int32 out, as spec_verify_run; lse_q [B, gamma] out or NULL;
 *   diag as spec_verify_run (lse_q entries are the sampler's normalisers).
 * Requires a context with max_rank == R; uses the context's Markov workspace. */
sv_status markov_verify_run(sv_ctx *ctx, hipStream_t stream,
                            const void *base_logits, const void *U, const void *Wt, int R,
                            const int32_t *x0, const void *p_logits, sv_dtype p_dtype,
                            int B, int gamma, int64_t V, float temperature,
                            uint64_t draft_seed, uint64_t verify_seed, uint64_t offset,
                            int32_t *draft_tokens, int32_t *accepted_len, int32_t *out_tokens,
                            float *lse_q, const sv_diag *diag);

/* RNN-head draft sampler ("DeepSeek DSpark 详解", section 03; "DSpark:
 * DeepSeek's bet on speed that doesn't betray quality", section "A drafter
 * that learns to doubt itself": a recurrent head keeps an in-block state and
 * so uses more of the prefix than the previous token; the pages give no
 * equations, and this is an Elman recurrence over the Markov head's
 * factors).  For k = 1..gamma, strictly
 * left to right, with h_0 = 0:
 *   a_k[j] = U[x_{k-1}, j] + sum_r A[j, r] hb_{k-1}[r]   (fp32, sequential
 *            fused multiply-adds over r = 0..R-1 starting from U[x_{k-1}, j])
 *   hb_k   = bf16(tanh(a_k))   (round to nearest, ties to even)
 *   z_k[n] = base_k[n] + sum_r hb_k[r] W[r, n]   (bf16 inputs, fp32 accumulation)
 *   x_k    = inverse-CDF draw from softmax(z_k / temperature), uniform tag 2.
 * With A = 0 it is the Markov head on bf16(tanh(U)).
 *   A             [R, R] bf16 device, 16-byte aligned, in a linear layer's
 *                 layout [out, in]: A[j, r] takes state entry r into entry j
 *   states        [B, gamma, R] bf16 out or NULL: hb_k, the state position k
 *                 used (not written for a request whose draw failed)
 *   other arguments as markov_draft_run.  With q_logits NULL no logit row is
 *   stored (the draw rebuilds the 64 logits of its chosen tile); the
 *   context's workspace holds the state between positions, so calls on one
 *   context must not overlap. */
sv_status rnn_draft_run(sv_ctx *ctx, hipStream_t stream,
                        const void *base_logits, const void *U, const void *Wt, const void *A, int R,
                        const int32_t *x0, int B, int gamma, int64_t V, float temperature,
                        uint64_t seed, uint64_t offset, const float *uniforms,
                        int32_t *draft_tokens, float *q_logits, float *lse_q, uint16_t *states);

/* ---- Measurement ------------------------------------------------------
 * Per-kernel timing with HIP events recorded on the caller's stream around
 * every kernel the library launches (the kernels themselves are unchanged).
 * For benchmarks and profiling only; off by default. */
typedef enum {
    SV_KERNEL_ROWSTATS = 0,      /* row statistics: one HBM pass over every verified row  */
    SV_KERNEL_ACCEPT = 1,        /* per-request acceptance scan / block thresholds        */
    SV_KERNEL_BLOCK_PASS2 = 2,   /* block verification residual masses                   */
    SV_KERNEL_RESID = 3,         /* correction / bonus weight sums per segment           */
    SV_KERNEL_SELECT = 4,        /* inverse-CDF draw of the correction / bonus token     */
    SV_KERNEL_TAIL = 5,          /* accept + weight sums + draw fused, one workgroup per request */
    SV_KERNEL_SCHEDULE = 6,      /* prefix scheduler                                     */
    SV_KERNEL_MARKOV_GEMM = 7,   /* Markov / RNN head contraction + epilogue (per position) */
    SV_KERNEL_MARKOV_SELECT = 8, /* Markov / RNN head draw (+ RNN state update), per position */
    SV_KERNEL_MARKOV_REBUILD = 9,/* fused path: correction rows rebuilt and weighed per tile */
    SV_KERNEL_COUNT = 10
} sv_kernel;

/* enable != 0 creates the context's event pool (up to 4096 launches per
 * read) and starts recording; 0 stops recording and frees the pool. */
sv_status spec_verify_profile_enable(sv_ctx *ctx, int enable);

/* Waits for the recorded events, writes per-kernel totals since the last read
 * (total_ms[SV_KERNEL_COUNT], launches[SV_KERNEL_COUNT], both host arrays) and
 * clears them.  Launches beyond the pool's capacity are not timed. */
sv_status spec_verify_profile_read(sv_ctx *ctx, double *total_ms, int64_t *launches);

#ifdef __cplusplus
}
#endif
#endif /* SPEC_VERIFY_H */
