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
 * q = p + N(0, 1), fp32; draft token i = the argmax of q row i.
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
    printf("C ABI parity: %d failures, %d within-margin flips\n", failures, flips);
    return failures ? 1 : 0;
}
