/*
 * c_abi_parity.c -- drives libspecverify.so through its C ABI alone (no
 * Python, no torch): device buffers from the HIP runtime, token-level and
 * block verification of a small seeded batch, then the same batch through the
 * CPU oracle (liboracle.so, test infrastructure).  Every decision must agree,
 * or differ only where the oracle reports a margin <= 1e-4 (a rounding flip).
 * Exit status 0 on success.
 *
 * Inputs (this file's own generator, shared by both sides): target logits
 * p ~ N(0, 3^2) with one token per row boosted by +6, draft logits
 * q = p + N(0, 1), fp32; draft token i = the argmax of q row i.  Then tree
 * verification of a small tree (rows generated the same way, each node's
 * token the argmax of its parent's draft row) and the prefix scheduler on
 * temperature-scaled confidence log-odds.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "oracle.h"
#include "spec_verify.h"

#define MARGIN 1e-4

static uint64_t rng = 0x9E3779B97F4A7C15ull;

static double uniform01(void)   /* xorshift64*, 53-bit uniform in (0, 1) */
{
    rng ^= rng >> 12;
    rng ^= rng << 25;
    rng ^= rng >> 27;
    const uint64_t x = rng * 0x2545F4914F6CDD1Dull;
    return ((double)(x >> 11) + 0.5) * (1.0 / 9007199254740992.0);
}

static double normal01(void)   /* Box-Muller */
{
    const double u1 = uniform01(), u2 = uniform01();
    return sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2);
}

#define CHECK_HIP(x)                                                                       \
    do {                                                                                   \
        hipError_t e_ = (x);                                                               \
        if (e_ != hipSuccess) {                                                            \
            fprintf(stderr, "HIP error %s at %s:%d\n", hipGetErrorString(e_), __FILE__, __LINE__); \
            return 2;                                                                      \
        }                                                                                  \
    } while (0)

#define CHECK_SV(x)                                                                        \
    do {                                                                                   \
        sv_status s_ = (x);                                                                \
        if (s_ != SV_OK) {                                                                 \
            fprintf(stderr, "library error %d: %s\n", (int)s_, spec_verify_last_error()); \
            return 2;                                                                      \
        }                                                                                  \
    } while (0)

/* Tree verification of a 6-node tree (root with children 1, 2, 5; node 1
 * with children 3, 4) through tree_verify_run against orc_tree_verify. */
static int tree_part(int *failures, int *flips)
{
    enum { B = 5, N = 5, NQ = 2 };
    const int32_t parents[N] = {0, 0, 1, 1, 0};
    const int D = 2;
    const int64_t V = 2003;
    const int qrow_of[N + 1] = {0, 1, -1, -1, -1, -1};   /* nodes with children: 0, 1 */
    const size_t np = (size_t)B * (N + 1) * V, nq = (size_t)B * NQ * V;
    float *p = malloc(np * sizeof(float)), *q = malloc(nq * sizeof(float));
    double *pd = malloc(np * sizeof(double)), *qd = malloc(nq * sizeof(double));
    int32_t tok[B * N];
    if (!p || !q || !pd || !qd) return 2;
    for (int b = 0; b < B; ++b) {
        for (int n = 0; n <= N; ++n) {
            float *row = p + ((size_t)b * (N + 1) + n) * V;
            for (int64_t v = 0; v < V; ++v) row[v] = (float)(3.0 * normal01());
            row[(int64_t)(uniform01() * V)] += 6.0f;
        }
        for (int n = 0; n <= N; ++n) {
            if (qrow_of[n] < 0) continue;
            const float *prow = p + ((size_t)b * (N + 1) + n) * V;
            float *qr = q + ((size_t)b * NQ + qrow_of[n]) * V;
            for (int64_t v = 0; v < V; ++v) qr[v] = prow[v] + (float)normal01();
        }
        for (int m = 1; m <= N; ++m) {   /* a token drawn from the parent's draft row (Gumbel-max) */
            const float *qr = q + ((size_t)b * NQ + qrow_of[parents[m - 1]]) * V;
            int64_t best = 0;
            double bv = -INFINITY;
            for (int64_t v = 0; v < V; ++v) {
                const double g = (double)qr[v] - log(-log(uniform01()));
                if (g > bv) { bv = g; best = v; }
            }
            tok[b * N + m - 1] = (int32_t)best;
        }
    }
    for (size_t k = 0; k < np; ++k) pd[k] = p[k];
    for (size_t k = 0; k < nq; ++k) qd[k] = q[k];

    void *dp, *dq, *dt, *dacc, *dout, *dnodes;
    CHECK_HIP(hipMalloc(&dp, np * sizeof(float)));
    CHECK_HIP(hipMalloc(&dq, nq * sizeof(float)));
    CHECK_HIP(hipMalloc(&dt, sizeof tok));
    CHECK_HIP(hipMalloc(&dacc, B * sizeof(int32_t)));
    CHECK_HIP(hipMalloc(&dout, (size_t)B * (D + 1) * sizeof(int32_t)));
    CHECK_HIP(hipMalloc(&dnodes, (size_t)B * D * sizeof(int32_t)));
    CHECK_HIP(hipMemcpy(dp, p, np * sizeof(float), hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dq, q, nq * sizeof(float), hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dt, tok, sizeof tok, hipMemcpyHostToDevice));
    sv_ctx *ctx = NULL;
    CHECK_SV(spec_verify_create(&ctx, 0, B, N, V, 0));
    CHECK_SV(tree_verify_run(ctx, 0, dp, SV_F32, dq, SV_F32, dt, parents, N, B, V, 1.0f, 11, 3, NULL, dacc, dout,
                             dnodes, NULL));
    uint32_t dev_flags = 0;
    CHECK_SV(spec_verify_device_status(ctx, 0, &dev_flags));
    int32_t gacc[B], gout[B * (D + 1)], gnodes[B * D];
    CHECK_HIP(hipMemcpy(gacc, dacc, sizeof gacc, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(gout, dout, sizeof gout, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(gnodes, dnodes, sizeof gnodes, hipMemcpyDeviceToHost));
    int32_t oacc[B], oout[B * (D + 1)], onodes[B * D];
    uint32_t ofl[B];
    double ratio[B * N], dm[B * N], im[B];
    if (orc_tree_verify(pd, qd, tok, parents, N, NULL, B, V, 1.0f, 11, 3, NULL, oacc, oout, onodes, ofl, ratio,
                        dm, im) != 0 || dev_flags != 0) {
        fprintf(stderr, "tree: oracle error or device flags %u\n", dev_flags);
        return 2;
    }
    for (int b = 0; b < B; ++b) {
        int same = gacc[b] == oacc[b];
        for (int j = 0; j <= D && same; ++j) same = gout[b * (D + 1) + j] == oout[b * (D + 1) + j];
        for (int j = 0; j < D && same; ++j) same = gnodes[b * D + j] == onodes[b * D + j];
        if (same) continue;
        /* a disagreement must sit on a decision the oracle took within 1e-4 */
        double mm = im[b];
        for (int m = 0; m < N; ++m)
            if (!isnan(dm[b * N + m]) && dm[b * N + m] < mm) mm = dm[b * N + m];
        if (mm <= MARGIN) {
            ++*flips;
        } else {
            fprintf(stderr, "tree b=%d: accepted %d (oracle %d)\n", b, gacc[b], oacc[b]);
            ++*failures;
        }
    }
    printf("tree verification through the C ABI: accepted =");
    for (int b = 0; b < B; ++b) printf(" %d", gacc[b]);
    printf("\n");
    spec_verify_destroy(ctx);
    (void)hipFree(dp); (void)hipFree(dq); (void)hipFree(dt);
    (void)hipFree(dacc); (void)hipFree(dout); (void)hipFree(dnodes);
    free(p); free(q); free(pd); free(qd);
    return 0;
}

/* The prefix scheduler on temperature-scaled confidence log-odds through
 * spec_schedule_sts_run against orc_sts_confidence + orc_schedule. */
static int schedule_part(int *failures, int *flips)
{
    enum { B = 40, G = 6 };
    float logits[B * G];
    const float temps[G] = {1.0f, 1.1f, 1.25f, 1.4f, 1.6f, 1.8f};
    double lg[B * G], td[G], conf[B * G];
    for (int k = 0; k < B * G; ++k) {
        logits[k] = (float)(1.2 + 1.5 * normal01());
        lg[k] = logits[k];
    }
    for (int i = 0; i < G; ++i) td[i] = temps[i];
    void *dl, *dvl, *dex;
    CHECK_HIP(hipMalloc(&dl, sizeof logits));
    CHECK_HIP(hipMalloc(&dvl, B * sizeof(int32_t)));
    CHECK_HIP(hipMalloc(&dex, sizeof(double)));
    CHECK_HIP(hipMemcpy(dl, logits, sizeof logits, hipMemcpyHostToDevice));
    sv_ctx *ctx = NULL;
    CHECK_SV(spec_verify_create(&ctx, 0, B, G, 16, 0));
    CHECK_SV(spec_schedule_sts_run(ctx, 0, dl, temps, B, G, 2000.0f, 50.0f, dvl, dex));
    int32_t gvl[B];
    double gex = 0.0;
    CHECK_HIP(hipMemcpy(gvl, dvl, sizeof gvl, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(&gex, dex, sizeof gex, hipMemcpyDeviceToHost));
    int32_t ovl[B];
    double oex = 0.0, margin = 0.0;
    if (orc_sts_confidence(lg, td, B, G, conf) != 0 || orc_schedule(conf, B, G, 2000.0, 50.0, ovl, &oex, &margin) != 0)
        return 2;
    int same = 1;
    for (int b = 0; b < B; ++b) same &= gvl[b] == ovl[b];
    if (!same) {
        if (margin <= 1e-12) ++*flips;
        else { fprintf(stderr, "scheduler: allocations differ (stop margin %.3e)\n", margin); ++*failures; }
    } else if (fabs(gex - oex) > 1e-12 * oex) {
        fprintf(stderr, "scheduler: expected %.17g vs oracle %.17g\n", gex, oex);
        ++*failures;
    }
    int tot = 0;
    for (int b = 0; b < B; ++b) tot += gvl[b];
    printf("temperature-scaled scheduler through the C ABI: %d positions admitted, E = %.6f\n", tot, gex);
    spec_verify_destroy(ctx);
    (void)hipFree(dl); (void)hipFree(dvl); (void)hipFree(dex);
    return 0;
}

int main(void)
{
    const int B = 6, gamma = 4;
    const int64_t V = 3001;
    const float T = 1.0f;
    const uint64_t seed = 1, offset = 7;
    const size_t np = (size_t)B * (gamma + 1) * V, nq = (size_t)B * gamma * V;

    float *p = malloc(np * sizeof(float)), *q = malloc(nq * sizeof(float));
    double *pd = malloc(np * sizeof(double)), *qd = malloc(nq * sizeof(double));
    int32_t *draft = malloc((size_t)B * gamma * sizeof(int32_t));
    if (!p || !q || !pd || !qd || !draft) return 2;
    for (int b = 0; b < B; ++b) {
        for (int i = 0; i <= gamma; ++i) {
            float *row = p + ((size_t)b * (gamma + 1) + i) * V;
            for (int64_t v = 0; v < V; ++v) row[v] = (float)(3.0 * normal01());
            row[(int64_t)(uniform01() * V)] += 6.0f;
        }
        for (int i = 0; i < gamma; ++i) {
            const float *prow = p + ((size_t)b * (gamma + 1) + i) * V;
            float *qrow = q + ((size_t)b * gamma + i) * V;
            int64_t best = 0;
            for (int64_t v = 0; v < V; ++v) {
                qrow[v] = prow[v] + (float)normal01();
                if (qrow[v] > qrow[best]) best = v;
            }
            draft[b * gamma + i] = (int32_t)best;
        }
    }
    for (size_t k = 0; k < np; ++k) pd[k] = p[k];
    for (size_t k = 0; k < nq; ++k) qd[k] = q[k];

    void *dp, *dq, *dx, *dacc, *dout;
    CHECK_HIP(hipMalloc(&dp, np * sizeof(float)));
    CHECK_HIP(hipMalloc(&dq, nq * sizeof(float)));
    CHECK_HIP(hipMalloc(&dx, (size_t)B * gamma * sizeof(int32_t)));
    CHECK_HIP(hipMalloc(&dacc, (size_t)B * sizeof(int32_t)));
    CHECK_HIP(hipMalloc(&dout, (size_t)B * (gamma + 1) * sizeof(int32_t)));
    CHECK_HIP(hipMemcpy(dp, p, np * sizeof(float), hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dq, q, nq * sizeof(float), hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dx, draft, (size_t)B * gamma * sizeof(int32_t), hipMemcpyHostToDevice));

    sv_ctx *ctx = NULL;
    CHECK_SV(spec_verify_create(&ctx, 0, B, gamma, V, 0));

    int failures = 0, flips = 0;
    for (int block = 0; block <= 1; ++block) {
        if (block)
            CHECK_SV(spec_blockverify_run(ctx, 0, dp, SV_F32, dq, SV_F32, dx, NULL, NULL, 0.0f, 0.0f, NULL, B, gamma,
                                          V, T, seed, offset, NULL, dacc, dout, NULL));
        else
            CHECK_SV(spec_verify_run(ctx, 0, dp, SV_F32, dq, SV_F32, dx, NULL, B, gamma, V, T, seed, offset, NULL,
                                     dacc, dout, NULL));
        uint32_t dev_flags = 0;
        CHECK_SV(spec_verify_device_status(ctx, 0, &dev_flags));
        int32_t gacc[64], gout[64 * 8];
        CHECK_HIP(hipMemcpy(gacc, dacc, (size_t)B * sizeof(int32_t), hipMemcpyDeviceToHost));
        CHECK_HIP(hipMemcpy(gout, dout, (size_t)B * (gamma + 1) * sizeof(int32_t), hipMemcpyDeviceToHost));

        int32_t oacc[64], oout[64 * 8];
        uint32_t oflags[64];
        double dec_margin[64 * 8], icdf_margin[64];
        orc_diag diag;
        memset(&diag, 0, sizeof(diag));
        diag.dec_margin = dec_margin;
        diag.icdf_margin = icdf_margin;
        const int rc = block ? orc_block_verify(pd, qd, draft, NULL, NULL, B, gamma, V, T, seed, offset, NULL,
                                                oacc, oout, oflags, &diag)
                             : orc_token_verify(pd, qd, draft, NULL, NULL, B, gamma, V, T, seed, offset, NULL,
                                                oacc, oout, oflags, &diag);
        if (rc != 0 || dev_flags != 0) {
            fprintf(stderr, "oracle rc %d, device flags %u\n", rc, dev_flags);
            return 1;
        }
        for (int b = 0; b < B; ++b) {
            const int oa = oacc[b], ga = gacc[b];
            if (oa != ga) {
                const int i = block ? (oa > ga ? oa : ga) - 1 : (oa < ga ? oa : ga);
                if (dec_margin[b * gamma + i] <= MARGIN) {
                    ++flips;
                } else {
                    fprintf(stderr, "%s b=%d: accepted %d (oracle %d), margin %.3e\n", block ? "block" : "token", b,
                            ga, oa, dec_margin[b * gamma + i]);
                    ++failures;
                }
                continue;
            }
            for (int j = 0; j <= gamma; ++j) {
                const int32_t o = oout[b * (gamma + 1) + j], g = gout[b * (gamma + 1) + j];
                if (o == g) continue;
                if (j == oa && icdf_margin[b] <= MARGIN) {
                    ++flips;
                } else {
                    fprintf(stderr, "%s b=%d: token %d is %d (oracle %d)\n", block ? "block" : "token", b, j, g, o);
                    ++failures;
                }
                break;
            }
        }
        printf("%s verification through the C ABI: accepted =", block ? "block" : "token");
        for (int b = 0; b < B; ++b) printf(" %d", gacc[b]);
        printf("\n");
    }
    spec_verify_destroy(ctx);
    (void)hipFree(dp);
    (void)hipFree(dq);
    (void)hipFree(dx);
    (void)hipFree(dacc);
    (void)hipFree(dout);
    free(p); free(q); free(pd); free(qd); free(draft);

    if (tree_part(&failures, &flips) != 0) return 2;
    if (schedule_part(&failures, &flips) != 0) return 2;
    printf("C ABI parity: %d failures, %d within-margin flips\n", failures, flips);
    return failures ? 1 : 0;
}
