/*
 * oracle.c -- plain, slow CPU reference for lossless speculative-sampling
 * verification.  TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check
 * and the benchmark's CPU-baseline leg, never by the GPU library, with which
 * it shares no code.  Definitions, sources and conventions: oracle.h.
 *
 * Every loop runs in index order; every sum is sequential binary64.
 * Decisions compare in binary32 (the GPU's precision); margins are binary64.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------- */
/* Philox4x32-10, from the definition in Salmon et al., SC'11, section 3:     */
/* the Philox S-box multiplies two of the four words by fixed 32-bit          */
/* multipliers, XORs the high halves of the products into the other two words */
/* and the round key, and permutes the words; the 2-word key advances by the  */
/* Weyl constants between rounds; ten rounds.                                 */
/* ------------------------------------------------------------------------- */
void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;   /* multipliers       */
    const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;   /* key Weyl steps    */
    uint32_t x0 = ctr[0], x1 = ctr[1], x2 = ctr[2], x3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        uint64_t prod0 = (uint64_t)M0 * (uint64_t)x0;
        uint64_t prod1 = (uint64_t)M1 * (uint64_t)x2;
        uint32_t hi0 = (uint32_t)(prod0 >> 32), lo0 = (uint32_t)prod0;
        uint32_t hi1 = (uint32_t)(prod1 >> 32), lo1 = (uint32_t)prod1;
        uint32_t y0 = hi1 ^ x1 ^ k0;
        uint32_t y1 = lo1;
        uint32_t y2 = hi0 ^ x3 ^ k1;
        uint32_t y3 = lo0;
        x0 = y0; x1 = y1; x2 = y2; x3 = y3;
        k0 += W0;
        k1 += W1;
    }
    out[0] = x0; out[1] = x1; out[2] = x2; out[3] = x3;
}

float orc_uniform(uint64_t seed, uint64_t offset, uint32_t req, uint32_t pos, uint32_t tag)
{
    uint32_t key[2] = { (uint32_t)seed, (uint32_t)(seed >> 32) };
    uint32_t ctr[4] = { req, (pos & 0xFFFFu) | (tag << 16),
                        (uint32_t)offset, (uint32_t)(offset >> 32) };
    uint32_t out[4];
    orc_philox4x32_10(ctr, key, out);
    /* 24 high bits scaled by 2^-24: every value is exact in binary32. */
    return (float)((double)(out[0] >> 8) * (1.0 / 16777216.0));
}

/* ------------------------------------------------------------------------- */
/* Softmax normaliser of one row: lse = log sum_v exp(z_v), z_v = row_v / T.  */
/* Needed because the acceptance rule and the residual work on normalised     */
/* probabilities p(x), q(x) ("The rule that makes it exact").                 */
/* ------------------------------------------------------------------------- */
uint32_t orc_row_lse(const double *row, int64_t V, float temperature, double *lse)
{
    const double T = (double)temperature;
    double m = -INFINITY;
    for (int64_t v = 0; v < V; ++v) {
        double x = row[v];
        if (isnan(x) || x == INFINITY) return ORC_FLAG_BAD_ROW;
        double z = x / T;
        if (z > m) m = z;
    }
    if (m == -INFINITY) return ORC_FLAG_BAD_ROW;
    double s = 0.0;
    for (int64_t v = 0; v < V; ++v) s += exp(row[v] / T - m);
    *lse = m + log(s);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Inverse-CDF draw: smallest v whose cumulative weight exceeds u * Z.        */
/* ------------------------------------------------------------------------- */
int64_t orc_icdf(const double *w, int64_t V, float u, double *Z_out, double *margin_out)
{
    double Z = 0.0;
    int64_t last = -1;
    for (int64_t v = 0; v < V; ++v) {
        Z += w[v];
        if (w[v] > 0.0) last = v;
    }
    if (Z_out) *Z_out = Z;
    if (last < 0) {
        if (margin_out) *margin_out = 0.0;
        return -1;
    }
    const float Zf = (float)Z;
    const float tf = (float)((double)u * (double)Zf);   /* u*Z rounded once to binary32 */
    const double t = (double)u * Z;
    double C = 0.0, Cprev = 0.0;
    int64_t y = -1;
    for (int64_t v = 0; v < V; ++v) {
        Cprev = C;
        C += w[v];
        if (w[v] > 0.0 && (float)C > tf) { y = v; break; }
    }
    if (y < 0) {                       /* t rounded up to Z: take the last token with weight */
        y = last;
        C = Z;
        Cprev = Z - w[last];
    }
    if (margin_out) {
        double a = t - Cprev, b = C - t;
        *margin_out = (a < b ? a : b) / Z;
    }
    return y;
}

/* ------------------------------------------------------------------------- */
/* Shared per-request preparation for token and block verification.          */
/* ------------------------------------------------------------------------- */
static void put_diag_nan(const orc_diag *d, int b, int gamma)
{
    if (!d) return;
    for (int i = 0; i < gamma; ++i) {
        if (d->ratio) d->ratio[(int64_t)b * gamma + i] = NAN;
        if (d->w) d->w[(int64_t)b * gamma + i] = NAN;
        if (d->h) d->h[(int64_t)b * gamma + i] = NAN;
        if (d->m) d->m[(int64_t)b * gamma + i] = NAN;
        if (d->dec_margin) d->dec_margin[(int64_t)b * gamma + i] = NAN;
        if (d->lse_q) d->lse_q[(int64_t)b * gamma + i] = NAN;
    }
    for (int i = 0; i <= gamma; ++i) {
        if (d->lse_p) d->lse_p[(int64_t)b * (gamma + 1) + i] = NAN;
        if (d->uniform) d->uniform[(int64_t)b * (gamma + 1) + i] = NAN;
    }
    if (d->resid_mass) d->resid_mass[b] = NAN;
    if (d->icdf_margin) d->icdf_margin[b] = NAN;
}

/* Validates tokens 1..L and normalises p rows 1..L+1 and q rows 1..L.
 * Returns the request's flags (0 = usable). */
static uint32_t prepare_request(const double *pb, const double *qb, const int32_t *xb,
                                int L, int64_t V, float T, double *lse_p, double *lse_q)
{
    uint32_t fl = 0;
    for (int i = 1; i <= L; ++i)
        if (xb[i - 1] < 0 || (int64_t)xb[i - 1] >= V) fl |= ORC_FLAG_BAD_TOKEN;
    if (fl) return fl;
    for (int i = 1; i <= L + 1; ++i) fl |= orc_row_lse(pb + (int64_t)(i - 1) * V, V, T, &lse_p[i]);
    for (int i = 1; i <= L; ++i) fl |= orc_row_lse(qb + (int64_t)(i - 1) * V, V, T, &lse_q[i]);
    return fl;
}

/* p(x_i) / q(x_i) at draft position i (1-based), in log space so that
 * neither probability underflows.  q(x)=0 < p(x) gives +inf (always accept);
 * p(x)=0 gives 0 (never accept); both 0 gives 0. */
static double target_draft_ratio(const double *pb, const double *qb, int i, int32_t x,
                                 int64_t V, double T, const double *lse_p, const double *lse_q)
{
    double lp = pb[(int64_t)(i - 1) * V + x] / T - lse_p[i];
    double lq = qb[(int64_t)(i - 1) * V + x] / T - lse_q[i];
    double r = exp(lp - lq);
    return isnan(r) ? 0.0 : r;
}

static float draw(const float *uniforms, int b, int gamma, int col, uint64_t seed,
                  uint64_t offset, uint32_t req, uint32_t pos, uint32_t tag)
{
    if (uniforms) return uniforms[(int64_t)b * (gamma + 1) + col];
    return orc_uniform(seed, offset, req, pos, tag);
}

static int check_common(const double *p, const double *q, const int32_t *draft, int B,
                        int gamma, int64_t V, float temperature, const int32_t *accepted_len,
                        const int32_t *out_tokens)
{
    if (B < 0 || gamma < 0 || V <= 0) return -1;
    if (!(temperature > 0.0f) || !isfinite(temperature)) return -1;
    if (B > 0 && (!p || !accepted_len || !out_tokens)) return -1;
    if (B > 0 && gamma > 0 && (!q || !draft)) return -1;
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Token-level verification ("The loop" and "The rule that makes it exact"): */
/* walk the draft left to right, accept x_i with probability                  */
/* min(1, p(x_i)/q(x_i)), stop at the first rejection; on a rejection at      */
/* position tau+1 draw the correction from max(p - q, 0) normalised; if all   */
/* L positions pass, draw the bonus token from p at position L+1.             */
/* ------------------------------------------------------------------------- */
int orc_token_verify(const double *p, const double *q, const int32_t *draft,
                     const int32_t *verify_len, const int32_t *req_ids,
                     int B, int gamma, int64_t V, float temperature,
                     uint64_t seed, uint64_t offset, const float *uniforms,
                     int32_t *accepted_len, int32_t *out_tokens, uint32_t *flags,
                     const orc_diag *d)
{
    if (check_common(p, q, draft, B, gamma, V, temperature, accepted_len, out_tokens)) return -1;
    for (int b = 0; b < B; ++b)
        if (verify_len && (verify_len[b] < 0 || verify_len[b] > gamma)) return -1;
    const double T = (double)temperature;
    double *wv = (double *)malloc((size_t)V * sizeof(double));
    double *lse_p = (double *)malloc((size_t)(gamma + 2) * sizeof(double));
    double *lse_q = (double *)malloc((size_t)(gamma + 2) * sizeof(double));
    if (!wv || !lse_p || !lse_q) { free(wv); free(lse_p); free(lse_q); return -1; }

    for (int b = 0; b < B; ++b) {
        const uint32_t req = req_ids ? (uint32_t)req_ids[b] : (uint32_t)b;
        const int L = verify_len ? verify_len[b] : gamma;
        const double *pb = p + (int64_t)b * (gamma + 1) * V;
        const double *qb = gamma > 0 ? q + (int64_t)b * gamma * V : NULL;
        const int32_t *xb = gamma > 0 ? draft + (int64_t)b * gamma : NULL;
        for (int j = 0; j <= gamma; ++j) out_tokens[(int64_t)b * (gamma + 1) + j] = -1;
        put_diag_nan(d, b, gamma);

        uint32_t fl = prepare_request(pb, qb, xb, L, V, temperature, lse_p, lse_q);
        if (flags) flags[b] = fl;
        if (fl) { accepted_len[b] = -1; continue; }
        if (d) {
            for (int i = 1; i <= L + 1; ++i)
                if (d->lse_p) d->lse_p[(int64_t)b * (gamma + 1) + i - 1] = lse_p[i];
            for (int i = 1; i <= L; ++i)
                if (d->lse_q) d->lse_q[(int64_t)b * gamma + i - 1] = lse_q[i];
        }

        int tau = L;
        for (int i = 1; i <= L; ++i) {
            double r = target_draft_ratio(pb, qb, i, xb[i - 1], V, T, lse_p, lse_q);
            double ratio = r < 1.0 ? r : 1.0;
            float u = draw(uniforms, b, gamma, i - 1, seed, offset, req, (uint32_t)i, 0);
            if (d && d->ratio) d->ratio[(int64_t)b * gamma + i - 1] = ratio;
            if (d && d->dec_margin) d->dec_margin[(int64_t)b * gamma + i - 1] = fabs((double)u - ratio);
            if (d && d->uniform) d->uniform[(int64_t)b * (gamma + 1) + i - 1] = u;
            if (!(u < (float)ratio)) { tau = i - 1; break; }
        }

        /* Correction (tau < L) or bonus (tau == L) weights over row tau+1. */
        const double *pr = pb + (int64_t)tau * V;
        const double lp = lse_p[tau + 1];
        if (tau < L) {
            const double *qr = qb + (int64_t)tau * V;
            const double lq = lse_q[tau + 1];
            for (int64_t v = 0; v < V; ++v) {
                double diff = exp(pr[v] / T - lp) - exp(qr[v] / T - lq);
                wv[v] = diff > 0.0 ? diff : 0.0;
            }
        } else {
            for (int64_t v = 0; v < V; ++v) wv[v] = exp(pr[v] / T - lp);
        }
        float u2 = draw(uniforms, b, gamma, gamma, seed, offset, req, 0, 1);
        double Z = 0.0, marg = 0.0;
        int64_t y = orc_icdf(wv, V, u2, &Z, &marg);
        if (y < 0) {
            /* The residual's mass rounded to zero (in exact arithmetic a
             * rejection implies p != q, so Z > 0): fall back to p. */
            for (int64_t v = 0; v < V; ++v) wv[v] = exp(pr[v] / T - lp);
            y = orc_icdf(wv, V, u2, &Z, &marg);
            fl |= ORC_FLAG_RESID_ZERO;
            if (flags) flags[b] = fl;
        }
        if (d && d->uniform) d->uniform[(int64_t)b * (gamma + 1) + gamma] = u2;
        if (d && d->resid_mass) d->resid_mass[b] = Z;
        if (d && d->icdf_margin) d->icdf_margin[b] = marg;

        accepted_len[b] = tau;
        for (int j = 0; j < tau; ++j) out_tokens[(int64_t)b * (gamma + 1) + j] = xb[j];
        out_tokens[(int64_t)b * (gamma + 1) + tau] = (int32_t)y;
    }
    free(wv); free(lse_p); free(lse_q);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Block verification ("Block verification", luminal page).  The page fixes  */
/* the running ratio w_i = min(1, w_{i-1} * p(x_i)/q(x_i)) with w_0 = 1, that */
/* the longest passing prefix is kept, and that separate thresholds and a     */
/* correction keep the output distributed as p.  Completion used here:       */
/*   m_i = sum_v max(w_i p_{i+1}(v) - q_{i+1}(v), 0)            (i < L)       */
/*   h_i = m_i / (m_i + 1 - w_i)   (h_i = 1 when that is 0/0)   (i < L)       */
/*   h_L = w_L                                                                */
/*   tau = largest i in 1..L with eta_i < h_i, else 0                         */
/*   y ~ p_{L+1} if tau = L, else max(w_tau p_{tau+1} - q_{tau+1}, 0).        */
/* With L = 1 this is token verification decision for decision.              */
/* ------------------------------------------------------------------------- */
int orc_block_verify(const double *p, const double *q, const int32_t *draft,
                     const int32_t *verify_len, const int32_t *req_ids,
                     int B, int gamma, int64_t V, float temperature,
                     uint64_t seed, uint64_t offset, const float *uniforms,
                     int32_t *accepted_len, int32_t *out_tokens, uint32_t *flags,
                     const orc_diag *d)
{
    if (check_common(p, q, draft, B, gamma, V, temperature, accepted_len, out_tokens)) return -1;
    for (int b = 0; b < B; ++b)
        if (verify_len && (verify_len[b] < 0 || verify_len[b] > gamma)) return -1;
    const double T = (double)temperature;
    double *wv = (double *)malloc((size_t)V * sizeof(double));
    double *lse_p = (double *)malloc((size_t)(gamma + 2) * sizeof(double));
    double *lse_q = (double *)malloc((size_t)(gamma + 2) * sizeof(double));
    double *w = (double *)malloc((size_t)(gamma + 2) * sizeof(double));
    double *h = (double *)malloc((size_t)(gamma + 2) * sizeof(double));
    if (!wv || !lse_p || !lse_q || !w || !h) {
        free(wv); free(lse_p); free(lse_q); free(w); free(h);
        return -1;
    }

    for (int b = 0; b < B; ++b) {
        const uint32_t req = req_ids ? (uint32_t)req_ids[b] : (uint32_t)b;
        const int L = verify_len ? verify_len[b] : gamma;
        const double *pb = p + (int64_t)b * (gamma + 1) * V;
        const double *qb = gamma > 0 ? q + (int64_t)b * gamma * V : NULL;
        const int32_t *xb = gamma > 0 ? draft + (int64_t)b * gamma : NULL;
        for (int j = 0; j <= gamma; ++j) out_tokens[(int64_t)b * (gamma + 1) + j] = -1;
        put_diag_nan(d, b, gamma);

        uint32_t fl = prepare_request(pb, qb, xb, L, V, temperature, lse_p, lse_q);
        if (flags) flags[b] = fl;
        if (fl) { accepted_len[b] = -1; continue; }
        if (d) {
            for (int i = 1; i <= L + 1; ++i)
                if (d->lse_p) d->lse_p[(int64_t)b * (gamma + 1) + i - 1] = lse_p[i];
            for (int i = 1; i <= L; ++i)
                if (d->lse_q) d->lse_q[(int64_t)b * gamma + i - 1] = lse_q[i];
        }

        /* Running capped ratio. */
        w[0] = 1.0;
        for (int i = 1; i <= L; ++i) {
            double r = target_draft_ratio(pb, qb, i, xb[i - 1], V, T, lse_p, lse_q);
            double ratio = r < 1.0 ? r : 1.0;
            double prod = (w[i - 1] == 0.0) ? 0.0 : w[i - 1] * r;   /* 0 * inf := 0 */
            w[i] = prod < 1.0 ? prod : 1.0;
            if (d && d->ratio) d->ratio[(int64_t)b * gamma + i - 1] = ratio;
            if (d && d->w) d->w[(int64_t)b * gamma + i - 1] = w[i];
        }
        /* Thresholds. */
        for (int i = 1; i < L; ++i) {
            const double *pn = pb + (int64_t)i * V;     /* p row i+1 */
            const double *qn = qb + (int64_t)i * V;     /* q row i+1 */
            double m = 0.0;
            for (int64_t v = 0; v < V; ++v) {
                double diff = w[i] * exp(pn[v] / T - lse_p[i + 1]) - exp(qn[v] / T - lse_q[i + 1]);
                if (diff > 0.0) m += diff;
            }
            double den = m + 1.0 - w[i];
            h[i] = den > 0.0 ? m / den : 1.0;
            if (d && d->m) d->m[(int64_t)b * gamma + i - 1] = m;
        }
        if (L >= 1) h[L] = w[L];

        int tau = 0;
        for (int i = 1; i <= L; ++i) {
            float eta = draw(uniforms, b, gamma, i - 1, seed, offset, req, (uint32_t)i, 0);
            if (d && d->h) d->h[(int64_t)b * gamma + i - 1] = h[i];
            if (d && d->dec_margin) d->dec_margin[(int64_t)b * gamma + i - 1] = fabs((double)eta - h[i]);
            if (d && d->uniform) d->uniform[(int64_t)b * (gamma + 1) + i - 1] = eta;
            if (eta < (float)h[i]) tau = i;
        }

        const double *pr = pb + (int64_t)tau * V;
        const double lp = lse_p[tau + 1];
        if (tau < L) {
            const double *qr = qb + (int64_t)tau * V;
            const double lq = lse_q[tau + 1];
            for (int64_t v = 0; v < V; ++v) {
                double diff = w[tau] * exp(pr[v] / T - lp) - exp(qr[v] / T - lq);
                wv[v] = diff > 0.0 ? diff : 0.0;
            }
        } else {
            for (int64_t v = 0; v < V; ++v) wv[v] = exp(pr[v] / T - lp);
        }
        float u2 = draw(uniforms, b, gamma, gamma, seed, offset, req, 0, 1);
        double Z = 0.0, marg = 0.0;
        int64_t y = orc_icdf(wv, V, u2, &Z, &marg);
        if (y < 0) {
            for (int64_t v = 0; v < V; ++v) wv[v] = exp(pr[v] / T - lp);
            y = orc_icdf(wv, V, u2, &Z, &marg);
            fl |= ORC_FLAG_RESID_ZERO;
            if (flags) flags[b] = fl;
        }
        if (d && d->uniform) d->uniform[(int64_t)b * (gamma + 1) + gamma] = u2;
        if (d && d->resid_mass) d->resid_mass[b] = Z;
        if (d && d->icdf_margin) d->icdf_margin[b] = marg;

        accepted_len[b] = tau;
        for (int j = 0; j < tau; ++j) out_tokens[(int64_t)b * (gamma + 1) + j] = xb[j];
        out_tokens[(int64_t)b * (gamma + 1) + tau] = (int32_t)y;
    }
    free(wv); free(lse_p); free(lse_q); free(w); free(h);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Hardware-aware prefix scheduler ("The Third Ace"; zskr.cn section 04).     */
/* Survival of the prefix ending at (b, i) is the running product of the     */
/* conditional acceptance estimates.  Candidates are ranked globally by       */
/* survival and admitted one by one while E[emitted] * SPS(rows) rises;      */
/* the first candidate that would not raise it stops admission (early stop,   */
/* which keeps admission independent of the tokens themselves).  Every        */
/* request always verifies its correction/bonus row, so E starts at B and the */
/* verify batch at B rows ("the 1 is the correction or bonus token").        */
/* With SPS(n) = a / (1 + n/K): E' * SPS(n+1) > E * SPS(n)  <=>  s (K+n) > E. */
/* ------------------------------------------------------------------------- */
typedef struct { double s; int b; int i; } orc_cand;

static int cand_cmp(const void *pa, const void *pb)
{
    const orc_cand *a = (const orc_cand *)pa, *c = (const orc_cand *)pb;
    if (a->s > c->s) return -1;          /* survival descending */
    if (a->s < c->s) return 1;
    if (a->b != c->b) return a->b < c->b ? -1 : 1;   /* then request ascending */
    if (a->i != c->i) return a->i < c->i ? -1 : 1;   /* then position ascending */
    return 0;
}

int orc_schedule(const double *conf, int B, int gamma, double sps_a, double sps_k,
                 int32_t *verify_len, double *expected, double *stop_margin)
{
    if (B < 0 || gamma < 0 || (B > 0 && (!verify_len || (gamma > 0 && !conf)))) return -1;
    if (!(sps_a > 0.0) || !(sps_k > 0.0)) return -1;
    (void)sps_a;   /* a positive scale of SPS does not change the argmax */
    for (int64_t k = 0; k < (int64_t)B * gamma; ++k)
        if (!(conf[k] >= 0.0 && conf[k] <= 1.0)) return -1;
    const int64_t n = (int64_t)B * gamma;
    orc_cand *c = (orc_cand *)malloc((size_t)(n > 0 ? n : 1) * sizeof(orc_cand));
    if (!c) return -1;
    for (int b = 0; b < B; ++b) {
        double S = 1.0;
        for (int i = 1; i <= gamma; ++i) {
            S = S * conf[(int64_t)b * gamma + i - 1];
            c[(int64_t)b * gamma + i - 1].s = S;
            c[(int64_t)b * gamma + i - 1].b = b;
            c[(int64_t)b * gamma + i - 1].i = i;
        }
        verify_len[b] = 0;
    }
    qsort(c, (size_t)n, sizeof(orc_cand), cand_cmp);
    double E = (double)B;
    double rows = (double)B;
    double margin = INFINITY;
    for (int64_t k = 0; k < n; ++k) {
        double gain = c[k].s * (sps_k + rows);
        if (gain > E) {
            E += c[k].s;
            rows += 1.0;
            verify_len[c[k].b] = c[k].i;
        } else {
            margin = (E > 0.0) ? (E - gain) / E : 0.0;
            break;
        }
    }
    if (expected) *expected = E;
    if (stop_margin) *stop_margin = margin;
    free(c);
    return 0;
}

/* Sequential temperature scaling: the logistic of logit / T_i, per position */
/* i, written out in binary64.  A positive temperature divides the log-odds, */
/* so T_i > 1 pulls the estimate toward 1/2 and T_i < 1 away from it.        */
int orc_sts_confidence(const double *logits, const double *temps, int B, int gamma, double *conf)
{
    if (B < 0 || gamma < 0) return -1;
    if (B > 0 && gamma > 0 && (!logits || !temps || !conf)) return -1;
    for (int i = 0; i < gamma; ++i)
        if (!(temps[i] > 0.0) || !isfinite(temps[i])) return -1;
    for (int b = 0; b < B; ++b) {
        for (int i = 0; i < gamma; ++i) {
            const double l = logits[(int64_t)b * gamma + i];
            if (isnan(l)) return -1;
            const double odds = exp(-(l / temps[i]));      /* e^{-l/T} in [0, +inf] */
            conf[(int64_t)b * gamma + i] = 1.0 / (1.0 + odds);
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Markov-head draft sampler ("The First Ace"; zskr.cn section 03): the       */
/* parallel backbone gives base logits for every block position; going left  */
/* to right, a rank-R transition U[x_{k-1}] . W is added to position k's      */
/* logits and x_k is sampled from the result, so each draw sees the previous. */
/* ------------------------------------------------------------------------- */
int orc_markov_draft(const double *base, const double *U, const double *W, int R,
                     const int32_t *x0, const int32_t *req_ids,
                     int B, int gamma, int64_t V, float temperature,
                     uint64_t seed, uint64_t offset, const float *uniforms,
                     int32_t *draft, double *q_logits, double *lse_q,
                     double *margin, uint32_t *flags)
{
    if (B < 0 || gamma < 0 || V <= 0 || R <= 0) return -1;
    if (!(temperature > 0.0f) || !isfinite(temperature)) return -1;
    if (B > 0 && gamma > 0 && (!base || !U || !W || !x0 || !draft)) return -1;
    const double T = (double)temperature;
    double *z = (double *)malloc((size_t)V * sizeof(double));
    double *wv = (double *)malloc((size_t)V * sizeof(double));
    if (!z || !wv) { free(z); free(wv); return -1; }

    for (int b = 0; b < B; ++b) {
        const uint32_t req = req_ids ? (uint32_t)req_ids[b] : (uint32_t)b;
        uint32_t fl = 0;
        for (int k = 0; k < gamma; ++k) {
            draft[(int64_t)b * gamma + k] = -1;
            if (lse_q) lse_q[(int64_t)b * gamma + k] = NAN;
            if (margin) margin[(int64_t)b * gamma + k] = NAN;
        }
        int32_t prev = x0 ? x0[b] : 0;
        if (gamma > 0 && (prev < 0 || (int64_t)prev >= V)) fl |= ORC_FLAG_BAD_TOKEN;
        for (int k = 1; k <= gamma && !fl; ++k) {
            const double *bk = base + ((int64_t)b * gamma + (k - 1)) * V;
            const double *Ur = U + (int64_t)prev * R;
            for (int64_t v = 0; v < V; ++v) {
                double dsum = 0.0;
                for (int r = 0; r < R; ++r) dsum += Ur[r] * W[(int64_t)r * V + v];
                z[v] = bk[v] + dsum;
            }
            double lse;
            fl |= orc_row_lse(z, V, temperature, &lse);
            if (fl) break;
            for (int64_t v = 0; v < V; ++v) wv[v] = exp(z[v] / T - lse);
            float u = uniforms ? uniforms[(int64_t)b * gamma + (k - 1)]
                               : orc_uniform(seed, offset, req, (uint32_t)k, 2);
            double Z, marg;
            int64_t y = orc_icdf(wv, V, u, &Z, &marg);
            if (y < 0) { fl |= ORC_FLAG_BAD_ROW; break; }
            draft[(int64_t)b * gamma + (k - 1)] = (int32_t)y;
            if (q_logits) memcpy(q_logits + ((int64_t)b * gamma + (k - 1)) * V, z, (size_t)V * sizeof(double));
            if (lse_q) lse_q[(int64_t)b * gamma + (k - 1)] = lse;
            if (margin) margin[(int64_t)b * gamma + (k - 1)] = marg;
            prev = (int32_t)y;
        }
        if (flags) flags[b] = fl;
    }
    free(z); free(wv);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* RNN-head draft sampler ("DeepSeek DSpark 详解", section 03: a recurrent    */
/* head keeps an in-block state, so each draw can use more of the prefix      */
/* than the previous token alone).  The pages give no equations; the plain    */
/* reading taken here is an Elman recurrence with the Markov head's factors:  */
/*   h_0 = 0,  a_k = U[x_{k-1}] + A hb_{k-1},  h_k = tanh(a_k),               */
/*   hb_k = bf16(h_k),  z_k = base_k + hb_k . W,  x_k ~ softmax(z_k / T).     */
/* The state is a bf16 activation like the factors; rounding it is a          */
/* quantisation decision, taken in the kernels' precision: a_k accumulated    */
/* in binary32 by sequential fused multiply-adds over r = 0..R-1 starting     */
/* from U[x_{k-1}], tanh in binary32, then round-to-nearest-even to bf16.     */
/* A is stored as a linear layer's weight, [out, in]: A[j][r] takes state     */
/* entry r into entry j.  The contraction z_k is binary64 like the Markov     */
/* head's.                                                                    */
/* ------------------------------------------------------------------------- */

/* Round a binary32 value to the nearest bf16 (8 significant bits), ties to
 * even; *dist_ulps gets the distance from the rounding midpoint in binary32
 * units in the last place (0 = exactly halfway). */
static float orc_bf16_round(float x, double *dist_ulps)
{
    uint32_t u;
    memcpy(&u, &x, sizeof u);
    if ((u & 0x7F800000u) == 0x7F800000u) {   /* inf / NaN: unchanged */
        if (dist_ulps) *dist_ulps = INFINITY;
        return x;
    }
    const uint32_t low = u & 0xFFFFu;
    if (dist_ulps) *dist_ulps = fabs((double)low - 32768.0);
    uint32_t kept = u & 0xFFFF0000u;
    if (low > 0x8000u || (low == 0x8000u && (kept & 0x10000u))) kept += 0x10000u;   /* up in magnitude */
    float y;
    memcpy(&y, &kept, sizeof y);
    return y;
}

float orc_bf16(float x)
{
    return orc_bf16_round(x, NULL);
}

int orc_rnn_draft(const double *base, const double *U, const double *W, const double *A, int R,
                  const int32_t *x0, const int32_t *req_ids,
                  int B, int gamma, int64_t V, float temperature,
                  uint64_t seed, uint64_t offset, const float *uniforms,
                  int32_t *draft, double *q_logits, double *lse_q,
                  double *margin, uint32_t *flags, double *states, double *state_margin)
{
    if (B < 0 || gamma < 0 || V <= 0 || R <= 0) return -1;
    if (!(temperature > 0.0f) || !isfinite(temperature)) return -1;
    if (B > 0 && gamma > 0 && (!base || !U || !W || !A || !x0 || !draft)) return -1;
    const double T = (double)temperature;
    double *z = (double *)malloc((size_t)V * sizeof(double));
    double *wv = (double *)malloc((size_t)V * sizeof(double));
    float *hb = (float *)malloc((size_t)R * sizeof(float));
    float *hn = (float *)malloc((size_t)R * sizeof(float));
    if (!z || !wv || !hb || !hn) { free(z); free(wv); free(hb); free(hn); return -1; }

    for (int b = 0; b < B; ++b) {
        const uint32_t req = req_ids ? (uint32_t)req_ids[b] : (uint32_t)b;
        uint32_t fl = 0;
        for (int k = 0; k < gamma; ++k) {
            draft[(int64_t)b * gamma + k] = -1;
            if (lse_q) lse_q[(int64_t)b * gamma + k] = NAN;
            if (margin) margin[(int64_t)b * gamma + k] = NAN;
            if (state_margin) state_margin[(int64_t)b * gamma + k] = NAN;
        }
        for (int r = 0; r < R; ++r) hb[r] = 0.0f;            /* h_0 = 0 */
        int32_t prev = x0 ? x0[b] : 0;
        if (gamma > 0 && (prev < 0 || (int64_t)prev >= V)) fl |= ORC_FLAG_BAD_TOKEN;
        for (int k = 1; k <= gamma && !fl; ++k) {
            /* state update: a = U[x_{k-1}] + A hb_{k-1}, binary32 fma chain */
            double qmin = INFINITY;
            for (int j = 0; j < R; ++j) {
                float acc = (float)U[(int64_t)prev * R + j];
                for (int r = 0; r < R; ++r) acc = fmaf(hb[r], (float)A[(int64_t)j * R + r], acc);
                double d;
                hn[j] = orc_bf16_round(tanhf(acc), &d);
                if (d < qmin) qmin = d;
            }
            for (int j = 0; j < R; ++j) hb[j] = hn[j];
            if (states)
                for (int j = 0; j < R; ++j) states[((int64_t)b * gamma + (k - 1)) * R + j] = (double)hb[j];
            if (state_margin) state_margin[(int64_t)b * gamma + (k - 1)] = qmin;
            /* logits: z = base_k + hb_k . W */
            const double *bk = base + ((int64_t)b * gamma + (k - 1)) * V;
            for (int64_t v = 0; v < V; ++v) {
                double dsum = 0.0;
                for (int r = 0; r < R; ++r) dsum += (double)hb[r] * W[(int64_t)r * V + v];
                z[v] = bk[v] + dsum;
            }
            double lse;
            fl |= orc_row_lse(z, V, temperature, &lse);
            if (fl) break;
            for (int64_t v = 0; v < V; ++v) wv[v] = exp(z[v] / T - lse);
            float u = uniforms ? uniforms[(int64_t)b * gamma + (k - 1)]
                               : orc_uniform(seed, offset, req, (uint32_t)k, 2);
            double Z, marg;
            int64_t y = orc_icdf(wv, V, u, &Z, &marg);
            if (y < 0) { fl |= ORC_FLAG_BAD_ROW; break; }
            draft[(int64_t)b * gamma + (k - 1)] = (int32_t)y;
            if (q_logits) memcpy(q_logits + ((int64_t)b * gamma + (k - 1)) * V, z, (size_t)V * sizeof(double));
            if (lse_q) lse_q[(int64_t)b * gamma + (k - 1)] = lse;
            if (margin) margin[(int64_t)b * gamma + (k - 1)] = marg;
            prev = (int32_t)y;
        }
        if (flags) flags[b] = fl;
    }
    free(z); free(wv); free(hb); free(hn);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Tree verification ("Speculative Decoding: The Same Distribution, Twice as */
/* Fast", section 7: guess a tree of alternative continuations and check all */
/* of them in one pass).  The page gives no rule; the plain lossless reading */
/* is recursive rejection over the tree, whose children of a node are drawn  */
/* independently from the draft distribution q at that node:                 */
/*   at node n (starting at the root, 0) with residual r = p_n:              */
/*     for each child c of n in index order, token x:                        */
/*       accept with probability min(1, r(x) / q_n(x)); if accepted emit x   */
/*       and continue at c;                                                   */
/*       else r <- max(r - q_n, 0) normalised;                                */
/*     if every child was rejected, emit a draw from r and stop;             */
/*   at a leaf, emit a draw from p_leaf (the bonus token) and stop.          */
/* The first child's ratio is the token rule's, in log space; a chain-shaped */
/* tree is token verification decision for decision.                         */
/* ------------------------------------------------------------------------- */
int orc_tree_depth(const int32_t *parents, int N)
{
    if (N < 0 || (N > 0 && !parents)) return -1;
    int *dep = (int *)malloc((size_t)(N + 1) * sizeof(int));
    if (!dep) return -1;
    dep[0] = 0;
    int D = 0;
    for (int m = 1; m <= N; ++m) {
        const int32_t par = parents[m - 1];
        if (par < 0 || par >= m) { free(dep); return -1; }
        dep[m] = dep[par] + 1;
        if (dep[m] > D) D = dep[m];
    }
    free(dep);
    return D;
}

int orc_tree_verify(const double *p, const double *q, const int32_t *tokens, const int32_t *parents, int N,
                    const int32_t *req_ids, int B, int64_t V, float temperature,
                    uint64_t seed, uint64_t offset, const float *uniforms,
                    int32_t *accepted_len, int32_t *out_tokens, int32_t *accepted_nodes, uint32_t *flags,
                    double *ratio_out, double *dec_margin, double *icdf_margin)
{
    const int D = orc_tree_depth(parents, N);
    if (D < 0 || B < 0 || V <= 0) return -1;
    if (!(temperature > 0.0f) || !isfinite(temperature)) return -1;
    if (B > 0 && (!p || !accepted_len || !out_tokens || (N > 0 && (!q || !tokens)))) return -1;
    const double T = (double)temperature;
    /* q row of each internal node: its rank among the nodes with children */
    int *qrow = (int *)malloc((size_t)(N + 1) * sizeof(int));
    double *pd = (double *)malloc((size_t)V * sizeof(double));
    double *qd = (double *)malloc((size_t)V * sizeof(double));
    double *r = (double *)malloc((size_t)V * sizeof(double));
    double *lse_p = (double *)malloc((size_t)(N + 1) * sizeof(double));
    double *lse_q = (double *)malloc((size_t)(N + 1) * sizeof(double));
    if (!qrow || !pd || !qd || !r || !lse_p || !lse_q) {
        free(qrow); free(pd); free(qd); free(r); free(lse_p); free(lse_q);
        return -1;
    }
    int NQ = 0;
    for (int n = 0; n <= N; ++n) {
        qrow[n] = -1;
        for (int m = n + 1; m <= N; ++m)
            if (parents[m - 1] == n) { qrow[n] = NQ++; break; }
    }

    for (int b = 0; b < B; ++b) {
        const uint32_t req = req_ids ? (uint32_t)req_ids[b] : (uint32_t)b;
        const double *pb = p + (int64_t)b * (N + 1) * V;
        const double *qb = NQ > 0 ? q + (int64_t)b * NQ * V : NULL;
        const int32_t *xb = N > 0 ? tokens + (int64_t)b * N : NULL;
        for (int j = 0; j <= D; ++j) out_tokens[(int64_t)b * (D + 1) + j] = -1;
        if (accepted_nodes)
            for (int j = 0; j < D; ++j) accepted_nodes[(int64_t)b * D + j] = -1;
        for (int m = 0; m < N; ++m) {
            if (ratio_out) ratio_out[(int64_t)b * N + m] = NAN;
            if (dec_margin) dec_margin[(int64_t)b * N + m] = NAN;
        }
        if (icdf_margin) icdf_margin[b] = NAN;

        /* data errors: any token out of range, then any row */
        uint32_t fl = 0;
        for (int m = 0; m < N; ++m)
            if (xb[m] < 0 || (int64_t)xb[m] >= V) fl |= ORC_FLAG_BAD_TOKEN;
        if (!fl) {
            for (int n = 0; n <= N; ++n) fl |= orc_row_lse(pb + (int64_t)n * V, V, temperature, &lse_p[n]);
            for (int n = 0; n <= N; ++n)
                if (qrow[n] >= 0) fl |= orc_row_lse(qb + (int64_t)qrow[n] * V, V, temperature, &lse_q[n]);
        }
        if (flags) flags[b] = fl;
        if (fl) { accepted_len[b] = -1; continue; }

        int node = 0, depth = 0;
        int64_t y = -1;
        double Z = 0.0, marg = 0.0;
        for (;;) {
            const double *prow = pb + (int64_t)node * V;
            const double lp = lse_p[node];
            float u2 = uniforms ? uniforms[(int64_t)b * (N + 1) + N] : orc_uniform(seed, offset, req, 0, 1);
            if (qrow[node] < 0) {                       /* leaf: the bonus token from p */
                for (int64_t v = 0; v < V; ++v) r[v] = exp(prow[v] / T - lp);
                y = orc_icdf(r, V, u2, &Z, &marg);
                break;
            }
            const double *qr = qb + (int64_t)qrow[node] * V;
            const double lq = lse_q[node];
            for (int64_t v = 0; v < V; ++v) {
                pd[v] = exp(prow[v] / T - lp);
                qd[v] = exp(qr[v] / T - lq);
                r[v] = pd[v];                           /* residual weights; total Zr */
            }
            double Zr = 1.0;
            int accepted = -1, rejections = 0;
            for (int c = node + 1; c <= N; ++c) {
                if (parents[c - 1] != node) continue;
                const int32_t x = xb[c - 1];
                double rt;
                if (rejections == 0) {
                    const double lr = (prow[x] / T - lp) - (qr[x] / T - lq);
                    rt = exp(lr);
                    if (isnan(rt)) rt = 0.0;
                } else if (qd[x] > 0.0) {
                    rt = (r[x] / Zr) / qd[x];
                } else {
                    rt = r[x] > 0.0 ? INFINITY : 0.0;
                }
                const double ratio = rt < 1.0 ? rt : 1.0;
                float u = uniforms ? uniforms[(int64_t)b * (N + 1) + (c - 1)]
                                   : orc_uniform(seed, offset, req, (uint32_t)c, 0);
                if (ratio_out) ratio_out[(int64_t)b * N + (c - 1)] = ratio;
                if (dec_margin) dec_margin[(int64_t)b * N + (c - 1)] = fabs((double)u - ratio);
                if (u < (float)ratio) { accepted = c; break; }
                /* rejected: r <- max(r / Zr - q, 0), its total the next Zr */
                double Zn = 0.0;
                for (int64_t v = 0; v < V; ++v) {
                    double diff = r[v] / Zr - qd[v];
                    r[v] = diff > 0.0 ? diff : 0.0;
                    Zn += r[v];
                }
                if (Zn == 0.0) {   /* rounded to zero (positive in exact arithmetic): fall back to p */
                    for (int64_t v = 0; v < V; ++v) r[v] = pd[v];
                    Zn = 1.0;
                    fl |= ORC_FLAG_RESID_ZERO;
                }
                Zr = Zn;
                ++rejections;
            }
            if (accepted > 0) {
                out_tokens[(int64_t)b * (D + 1) + depth] = xb[accepted - 1];
                if (accepted_nodes) accepted_nodes[(int64_t)b * D + depth] = accepted;
                ++depth;
                node = accepted;
                continue;
            }
            y = orc_icdf(r, V, u2, &Z, &marg);          /* every child rejected: the residual */
            if (y < 0) {
                for (int64_t v = 0; v < V; ++v) r[v] = pd[v];
                y = orc_icdf(r, V, u2, &Z, &marg);
                fl |= ORC_FLAG_RESID_ZERO;
            }
            break;
        }
        if (flags) flags[b] = fl;
        if (icdf_margin) icdf_margin[b] = marg;
        accepted_len[b] = depth;
        out_tokens[(int64_t)b * (D + 1) + depth] = (int32_t)y;
    }
    free(qrow); free(pd); free(qd); free(r); free(lse_p); free(lse_q);
    return 0;
}
