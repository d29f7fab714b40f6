/*
 * oracle.h -- plain, slow CPU reference of lossless speculative-sampling
 * verification, block verification, the confidence prefix scheduler (with
 * temperature-scaled confidences), the Markov- and RNN-head draft samplers
 * and tree verification.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The GPU library never
 * includes, links or calls it, and it shares no code with the GPU library.
 *
 * Arithmetic is IEEE binary64 with a fixed, sequential (index-order)
 * summation, unless a comment says otherwise.  Where a floating-point value
 * decides an integer (accept/reject, inverse-CDF index) the comparison is taken
 * in binary32, the precision the GPU kernels decide in; the margin of every
 * such decision is reported in binary64 so that tests can tell a rounding
 * flip from a real disagreement.
 *
 * Sources (pages as published):
 *  [SD]  "Speculative Decoding: The Same Distribution, Twice as Fast"
 *        (derpx06.online explainer), sections 3 "The loop", 4 "The rule that
 *        makes it exact", 5 "What decides the speedup".
 *  [LU]  "How much does a token cost" (blog.luminal.com), sections
 *        "On Speculative Sampling", "Block verification", "Adaptive
 *        verification", "Our own simple cost model".
 *  [KC]  "DeepSeek Boosts Inference Speed by 85%..." (kongchang.com),
 *        sections "The First Ace", "The Second Ace", "The Third Ace".
 *  [ZS]  "DeepSeek DSpark 详解" (zskr.cn), sections 02-04 and Fig. 1.
 *  [AT]  "DSpark: DeepSeek's bet on speed that doesn't betray quality"
 *        (aitalk.it), section "Verifying only what matters".
 *  [PH]  Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as
 *        1, 2, 3", SC'11 -- the Philox4x32-10 generator.
 *
 * Conventions shared by every entry point:
 *  - Logits are given as binary64 arrays (bf16/fp32 inputs widen exactly).
 *  - Row layout: p is [B, gamma+1, V], q is [B, gamma, V], V innermost.
 *    q row i (1-based, i = 1..gamma) pairs with p row i; p row gamma+1 is the
 *    bonus row.
 *  - Temperature T: a row's distribution is softmax(logit / T).
 *  - Uniform for (request r, position i, tag t): see orc_uniform().
 *    Tags: 0 = acceptance test u_i / block threshold eta_i, 1 = correction or
 *    bonus draw u', 2 = Markov draft draw.
 *  - req_ids (nullable): the global request index used for the random
 *    counters of local request b; NULL means req_ids[b] = b.  It lets a test
 *    run the oracle on a sample of requests of a large batch.
 *  - Returned int: 0 on success, -1 on an invalid argument.  Data errors in a
 *    request (token id outside [0,V), a row that is all -inf or holds NaN or
 *    +inf) set bits in flags[b] and make accepted_len[b] = -1.
 */
#ifndef ORACLE_H
#define ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* flags[b] bits */
#define ORC_FLAG_BAD_TOKEN   1u  /* draft or anchor token outside [0, V) */
#define ORC_FLAG_BAD_ROW     2u  /* a needed row is all -inf, or holds NaN / +inf */
#define ORC_FLAG_RESID_ZERO  4u  /* residual mass rounded to 0; p row used instead */

/* Optional per-request diagnostics; every pointer may be NULL. */
typedef struct {
    double *lse_p;       /* [B, gamma+1] log-sum-exp of p rows (after 1/T)      */
    double *lse_q;       /* [B, gamma]   log-sum-exp of q rows                  */
    double *ratio;       /* [B, gamma]   min(1, p(x_i)/q(x_i)); NaN if unused    */
    double *w;           /* [B, gamma]   block: running capped ratio w_i        */
    double *h;           /* [B, gamma]   block: acceptance threshold h_i        */
    double *dec_margin;  /* [B, gamma]   |u_i - ratio_i| or |eta_i - h_i|       */
    double *resid_mass;  /* [B]          mass Z of the correction/bonus weights */
    double *icdf_margin; /* [B]          min(t - C(y-1), C(y) - t) / Z          */
    float  *uniform;     /* [B, gamma+1] uniforms used (col gamma = u')         */
    double *m;           /* [B, gamma]   block: residual mass m_i of position i < L
                                         (NaN elsewhere)                           */
} orc_diag;

/* Philox4x32-10 block function [PH]: out = bijection(key, ctr). */
void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);

/* Uniform in [0, 1 - 2^-24], exactly representable in binary32:
 * key = (seed lo32, seed hi32),
 * counter = (req, (pos & 0xFFFF) | (tag << 16), offset lo32, offset hi32),
 * u = (word0 >> 8) * 2^-24. */
float orc_uniform(uint64_t seed, uint64_t offset, uint32_t req, uint32_t pos, uint32_t tag);

/* Log-sum-exp of z = row / T over V entries.  Returns 0, or ORC_FLAG_BAD_ROW. */
uint32_t orc_row_lse(const double *row, int64_t V, float temperature, double *lse);

/* Inverse-CDF draw from non-negative weights w[0..V) with uniform u:
 * t = u * Z, y = smallest v with C(v) = sum_{x<=v} w_x > t (compared in
 * binary32), falling back to the last v with w_v > 0.  Returns y, or -1 if
 * every weight is 0.  *Z_out and *margin_out (nullable) get Z and the
 * relative CDF gap of the chosen index. */
int64_t orc_icdf(const double *w, int64_t V, float u, double *Z_out, double *margin_out);

/* Token-level verification [SD 3-4], [LU "On Speculative Sampling"].
 * verify_len (nullable, [B], each in [0, gamma]): positions checked per
 * request (gamma when NULL).  uniforms (nullable, [B, gamma+1]) replaces the
 * Philox draws: column i-1 is u_i, column gamma is u'.
 * Out: accepted_len[B] (tau_b), out_tokens[B, gamma+1] (x_1..x_tau, y, then -1),
 * flags[B] (nullable). */
int orc_token_verify(const double *p, const double *q, const int32_t *draft,
                     const int32_t *verify_len, const int32_t *req_ids,
                     int B, int gamma, int64_t V, float temperature,
                     uint64_t seed, uint64_t offset, const float *uniforms,
                     int32_t *accepted_len, int32_t *out_tokens, uint32_t *flags,
                     const orc_diag *diag);

/* Block verification [LU "Block verification"], completed as documented in
 * orc_block_verify's definition.  Same arguments and outputs as token
 * verification; with verify_len = 1 it takes the same decisions. */
int orc_block_verify(const double *p, const double *q, const int32_t *draft,
                     const int32_t *verify_len, const int32_t *req_ids,
                     int B, int gamma, int64_t V, float temperature,
                     uint64_t seed, uint64_t offset, const float *uniforms,
                     int32_t *accepted_len, int32_t *out_tokens, uint32_t *flags,
                     const orc_diag *diag);

/* Hardware-aware prefix scheduler [KC "The Third Ace"], [ZS 04].
 * conf [B, gamma] in [0, 1]: conditional acceptance estimates.
 * SPS(n) = sps_a / (1 + n / sps_k) steps/s for a verify batch of n rows.
 * Out: verify_len[B]; *expected (nullable) = E[emitted tokens] of the
 * chosen allocation; *stop_margin (nullable) = relative margin of the
 * decision that stopped admission (+inf if every candidate was admitted). */
int orc_schedule(const double *conf, int B, int gamma, double sps_a, double sps_k,
                 int32_t *verify_len, double *expected, double *stop_margin);

/* Sequential temperature scaling of the confidence head [KC "The Second
 * Ace"], [ZS 04], [AT "Verifying only what matters"]: the head gives, for
 * each request b and draft position i, a logit for "x_i passes given that
 * x_1..x_{i-1} passed"; position i has its own temperature T_i (fitted
 * offline on held-out data, left to right), and the calibrated estimate is
 * the logistic of the logit divided by T_i:
 *   conf[b, i] = 1 / (1 + exp(-logits[b, i] / temps[i])),   binary64.
 * Dividing by T_i > 0 keeps the order of the candidates of one position.
 * logits [B, gamma] (binary32 values), temps [gamma], each finite and > 0.
 * Out: conf [B, gamma].  Returns -1 on a NaN logit or an invalid
 * temperature. */
int orc_sts_confidence(const double *logits, const double *temps, int B, int gamma, double *conf);

/* Markov-head draft sampler [KC "The First Ace"], [ZS 03].
 * base [B, gamma, V] backbone logits, U [V, R], W [R, V], x0 [B] anchor tokens.
 * For k = 1..gamma: d = U[x_{k-1}, :] . W, z_k = base_k + d,
 * x_k ~ softmax(z_k / T) by inverse CDF with uniform (req, k, tag 2)
 * (uniforms [B, gamma] nullable overrides them).
 * Out: draft [B, gamma]; q_logits [B, gamma, V] (nullable) = z_k before 1/T;
 * lse_q [B, gamma] (nullable); margin [B, gamma] (nullable) = inverse-CDF
 * margins; flags [B] (nullable). */
int orc_markov_draft(const double *base, const double *U, const double *W, int R,
                     const int32_t *x0, const int32_t *req_ids,
                     int B, int gamma, int64_t V, float temperature,
                     uint64_t seed, uint64_t offset, const float *uniforms,
                     int32_t *draft, double *q_logits, double *lse_q,
                     double *margin, uint32_t *flags);

/* bf16 rounding (nearest, ties to even) of a binary32 value. */
float orc_bf16(float x);

/* RNN-head draft sampler [ZS 03] (the reading is in orc_rnn_draft's
 * definition): h_0 = 0; a_k = U[x_{k-1}] + A hb_{k-1} in binary32
 * (sequential fma over r from U[x_{k-1}]); hb_k = bf16(tanhf(a_k));
 * z_k = base_k + hb_k . W (binary64); x_k ~ softmax(z_k / T) by inverse CDF
 * with uniform (req, k, tag 2).  A [R, R] in linear-layer layout [out, in]:
 * A[j][r] takes state entry r into entry j.
 * Outputs as orc_markov_draft, plus states [B, gamma, R] (nullable) = hb_k
 * and state_margin [B, gamma] (nullable) = the smallest distance, in binary32
 * ulps, of any tanhf(a_k) entry from its bf16 rounding midpoint. */
int orc_rnn_draft(const double *base, const double *U, const double *W, const double *A, int R,
                  const int32_t *x0, const int32_t *req_ids,
                  int B, int gamma, int64_t V, float temperature,
                  uint64_t seed, uint64_t offset, const float *uniforms,
                  int32_t *draft, double *q_logits, double *lse_q,
                  double *margin, uint32_t *flags, double *states, double *state_margin);

/* Depth of a tree given by parents[m-1] in [0, m-1] for nodes m = 1..N
 * (node 0 is the root); -1 for an invalid tree. */
int orc_tree_depth(const int32_t *parents, int N);

/* Tree verification [SD 7] (the rule is in orc_tree_verify's definition):
 * recursive rejection over a token tree whose children of a node were drawn
 * independently from the draft distribution at that node.
 *   p [B, N+1, V]: row n = target logits after node n (row 0: the root);
 *   q [B, NQ, V]: draft logits at each node that has children, in node
 *   order (NQ = their number); tokens [B, N]: token of node m at column
 *   m-1; parents [N] (host): parent of node m, in [0, m-1].
 *   Uniforms: node c's test (req, c, tag 0), the final draw (req, 0, tag 1);
 *   uniforms [B, N+1] (nullable) overrides them (column c-1, column N).
 * Out (D = the tree's depth): accepted_len [B]; out_tokens [B, D+1] = the
 * accepted path's tokens, the drawn token, then -1; accepted_nodes [B, D]
 * (nullable) = the accepted nodes, then -1; flags [B] (nullable); ratio and
 * dec_margin [B, N] (nullable, NaN where unevaluated) = min(1, r(x)/q(x)) and
 * |u - ratio| of each evaluated node; icdf_margin [B] (nullable). */
int orc_tree_verify(const double *p, const double *q, const int32_t *tokens, const int32_t *parents, int N,
                    const int32_t *req_ids, int B, int64_t V, float temperature,
                    uint64_t seed, uint64_t offset, const float *uniforms,
                    int32_t *accepted_len, int32_t *out_tokens, int32_t *accepted_nodes, uint32_t *flags,
                    double *ratio_out, double *dec_margin, double *icdf_margin);

#ifdef __cplusplus
}
#endif
#endif /* ORACLE_H */
