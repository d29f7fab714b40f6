// verify.hip -- acceptance scan, block thresholds and the correction / bonus
// sampler of lossless speculative sampling.
//
// Token-level rule ("Speculative Decoding: The Same Distribution, Twice as
// Fast", sections 3-4): accept draft token x_i with probability
// min(1, p_i(x_i)/q_i(x_i)), walking left to right and stopping at the first
// rejection; after a rejection draw the correction from max(p - q, 0)
// normalised, after a full pass draw the bonus token from p.
//
// Block rule ("How much does a token cost", section "Block verification"):
// running capped ratio w_i = min(1, w_{i-1} p_i(x_i)/q_i(x_i)); every prefix
// gets its own threshold and the longest passing prefix is kept; completion
// used here (lossless, and equal to the token rule when one position is
// verified): m_i = sum_v max(w_i p_{i+1} - q_{i+1}, 0), h_i = m_i/(m_i+1-w_i)
// for i < L, h_L = w_L, tau = largest i with eta_i < h_i, correction from
// max(w_tau p_{tau+1} - q_{tau+1}, 0) or the bonus from p_{L+1}.
//
// Kernels (each hands its results to the next through global memory, so the
// only synchronisation is the kernel boundary):
//  k_accept       one wavefront per request: merges the row statistics into
//                 log-sum-exps, gathers the draft tokens' logits, draws the
//                 uniforms and decides tau (token rule, or block thresholds
//                 from the residual masses); also the block "pre" stage that
//                 only computes the running ratios.
//  k_block_pass2  grid (request, position i, chunk): partial sums of
//                 max(w_i p_{i+1} - q_{i+1}, 0).
//  k_resid_sum    grid (request, chunk): partial sums of the correction /
//                 bonus weights of row tau+1 (skipped when block pass 2
//                 already summed exactly those weights).
//  k_select       one workgroup per request: picks the chunk holding u * Z
//                 from the fp64 prefix of the chunk sums, then scans inside it
//                 for the token (inverse CDF in ascending token id order).
#include "sv_device.h"
#include "sv_internal.h"

namespace {

using svk::u32x4;

constexpr int NT = svh::kResidThreads;
constexpr int CHR = svh::kChunkR;
constexpr int MAXG = svh::kMaxGamma;
constexpr double kLn2d = 0.69314718055994530942;

enum Stage { STAGE_TOKEN = 0, STAGE_BLOCK_PRE = 1, STAGE_BLOCK_FINAL = 2 };

// Per-request result of k_accept, read by the kernels that follow.
struct ReqG {
    uint32_t flags;
    int32_t L;
    int32_t tau;
    int32_t mode;      // 0: residual weights max(wmul * p - q, 0), 1: bonus weights p
    float wmul;        // multiplier of p in the residual weights (w_tau; 1 for the token rule)
    float lp2, lq2;    // log2-sum-exp2 of p row tau+1 and q row tau+1
    float u2;          // correction / bonus uniform
};
static_assert(sizeof(ReqG) == svh::kReqStateBytes, "request state layout");

// log2 sum exp2 of a row from its chunk partials (fp64 result); flags a bad row.
__device__ double merge_row(const float2 *__restrict__ part, int64_t row, int nch1, bool &bad)
{
    const float2 *pr = part + row * nch1;
    float M = svk::neg_inf();
    for (int k = 0; k < nch1; ++k) M = fmaxf(M, pr[k].x);
    float S = 0.0f;
    if (M == svk::neg_inf()) {
        for (int k = 0; k < nch1; ++k) S += pr[k].y;   // 0, or NaN for a NaN element
    } else {
        for (int k = 0; k < nch1; ++k) S += pr[k].y * exp2f(pr[k].x - M);
    }
    if (!(S > 0.0f) || M == svk::pos_inf() || S == svk::pos_inf()) bad = true;
    return (double)M + log2((double)S);
}

// ---------------------------------------------------------------------------
// k_accept: one 64-thread workgroup per request.
// ---------------------------------------------------------------------------
template <int PES, int QES>
__global__ __launch_bounds__(svk::kWave) void k_accept(svh::VerifyArgs a, const float2 *__restrict__ part,
                                                       int nch1, const float *__restrict__ bm, int nchr,
                                                       int stage, ReqG *__restrict__ req,
                                                       float *__restrict__ lp2g, float *__restrict__ lq2g,
                                                       float *__restrict__ wrun,
                                                       uint32_t *__restrict__ errword)
{
    __shared__ double lp2[MAXG + 1];
    __shared__ double lq2[MAXG];
    __shared__ float rr[MAXG];
    const int b = blockIdx.x;
    const int lane = threadIdx.x;
    const int gamma = a.gamma;
    const int G1 = gamma + 1;
    const float nan = __builtin_nanf("");

    const int L = a.verify_len ? a.verify_len[b] : gamma;
    uint32_t flags = 0;
    if (L < 0 || L > gamma) flags = SV_FLAG_BAD_VERIFY_LEN;
    if (!flags) {   // tokens first: a bad token is reported alone
        bool badtok = false;
        for (int j = lane; j < L; j += svk::kWave) {
            const int32_t x = a.draft[(int64_t)b * gamma + j];
            if (x < 0 || (int64_t)x >= a.V) badtok = true;
        }
        if (__ballot(badtok)) flags = SV_FLAG_BAD_TOKEN;
    }
    const int64_t prow0 = (int64_t)b * G1;
    const int64_t qrow0 = (int64_t)a.B * G1 + (int64_t)b * gamma;
    if (!flags) {
        bool badrow = false;
        for (int j = lane; j <= L; j += svk::kWave) lp2[j] = merge_row(part, prow0 + j, nch1, badrow);
        for (int j = lane; j < L; j += svk::kWave) lq2[j] = merge_row(part, qrow0 + j, nch1, badrow);
        if (__ballot(badrow)) flags = SV_FLAG_BAD_ROW;
    }
    if (flags) {
        if (lane == 0) {
            ReqG r{};
            r.flags = flags;
            r.L = L;
            req[b] = r;
        }
        if (stage == STAGE_BLOCK_PRE) return;   // the final stage reports it
        for (int j = lane; j < G1; j += svk::kWave) {
            a.out_tokens[(int64_t)b * G1 + j] = -1;
            if (a.diag.lse_p) a.diag.lse_p[(int64_t)b * G1 + j] = nan;
        }
        for (int j = lane; j < gamma; j += svk::kWave) {
            if (a.diag.lse_q) a.diag.lse_q[(int64_t)b * gamma + j] = nan;
            if (a.diag.ratio) a.diag.ratio[(int64_t)b * gamma + j] = nan;
            if (a.diag.w) a.diag.w[(int64_t)b * gamma + j] = nan;
            if (a.diag.h) a.diag.h[(int64_t)b * gamma + j] = nan;
        }
        if (lane == 0) {
            a.accepted_len[b] = -1;
            if (a.diag.flags) a.diag.flags[b] = flags;
            if (a.diag.resid_mass) a.diag.resid_mass[b] = nan;
            atomicOr(errword, flags);
        }
        return;
    }

    // ratios of the draft tokens, log2 space, fp64
    for (int j = lane; j < L; j += svk::kWave) {
        const int32_t x = a.draft[(int64_t)b * gamma + j];
        const double xp = (double)svk::load_logit<PES>(a.p, (prow0 + j) * a.V + x) * (double)a.c;
        const double xq = (double)svk::load_logit<QES>(a.q, ((int64_t)b * gamma + j) * a.V + x) * (double)a.c;
        const float r = (float)exp2((xp - lp2[j]) - (xq - lq2[j]));
        rr[j] = (r != r) ? 0.0f : r;
    }
    // only this wavefront runs: order its LDS writes before lane 0 reads them
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    if (stage == STAGE_BLOCK_PRE) {
        for (int j = lane; j <= L; j += svk::kWave) lp2g[(int64_t)b * G1 + j] = (float)lp2[j];
        for (int j = lane; j < L; j += svk::kWave) lq2g[(int64_t)b * gamma + j] = (float)lq2[j];
        if (lane == 0) {
            float w = 1.0f;
            wrun[(int64_t)b * G1] = w;
            for (int i = 1; i <= L; ++i) {
                const float prod = w == 0.0f ? 0.0f : w * rr[i - 1];   // 0 * inf := 0
                w = fminf(prod, 1.0f);
                wrun[(int64_t)b * G1 + i] = w;
            }
            ReqG r{};
            r.flags = 0;
            r.L = L;
            req[b] = r;
        }
        return;
    }

    // diagnostics of the evaluated positions
    for (int j = lane; j < G1; j += svk::kWave)
        if (a.diag.lse_p) a.diag.lse_p[(int64_t)b * G1 + j] = j <= L ? (float)(lp2[j] * kLn2d) : nan;
    for (int j = lane; j < gamma; j += svk::kWave) {
        if (a.diag.lse_q) a.diag.lse_q[(int64_t)b * gamma + j] = j < L ? (float)(lq2[j] * kLn2d) : nan;
        if (a.diag.ratio) a.diag.ratio[(int64_t)b * gamma + j] = j < L ? fminf(rr[j], 1.0f) : nan;
    }
    if (lane != 0) return;

    const float u2 = a.uniforms ? a.uniforms[(int64_t)b * G1 + gamma]
                                : svk::philox_uniform(a.seed, a.offset, (uint32_t)b, 0u, 1u);
    int tau;
    float wmul = 1.0f;
    if (stage == STAGE_TOKEN) {
        tau = L;
        for (int j = 0; j < L; ++j) {
            const float ratio = fminf(rr[j], 1.0f);
            const float u = a.uniforms ? a.uniforms[(int64_t)b * G1 + j]
                                       : svk::philox_uniform(a.seed, a.offset, (uint32_t)b,
                                                             (uint32_t)(j + 1), 0u);
            if (!(u < ratio)) {
                tau = j;
                break;
            }
        }
        for (int i = 0; i < gamma; ++i) {
            if (a.diag.w) a.diag.w[(int64_t)b * gamma + i] = nan;
            if (a.diag.h) a.diag.h[(int64_t)b * gamma + i] = nan;
        }
    } else {
        // thresholds from the running ratios (block pre stage) and residual masses (pass 2)
        const float *w = wrun + (int64_t)b * G1;
        tau = 0;
        for (int i = 1; i <= L; ++i) {
            float h;
            if (i < L) {
                double m = 0.0;
                const float *bmi = bm + ((int64_t)b * gamma + i) * nchr;
                for (int k = 0; k < nchr; ++k) m += (double)bmi[k];
                const double den = m + 1.0 - (double)w[i];
                h = den > 0.0 ? (float)(m / den) : 1.0f;
            } else {
                h = w[L];
            }
            const float eta = a.uniforms ? a.uniforms[(int64_t)b * G1 + i - 1]
                                         : svk::philox_uniform(a.seed, a.offset, (uint32_t)b,
                                                               (uint32_t)i, 0u);
            if (eta < h) tau = i;
            if (a.diag.w) a.diag.w[(int64_t)b * gamma + i - 1] = w[i];
            if (a.diag.h) a.diag.h[(int64_t)b * gamma + i - 1] = h;
        }
        for (int i = L; i < gamma; ++i) {
            if (a.diag.w) a.diag.w[(int64_t)b * gamma + i] = nan;
            if (a.diag.h) a.diag.h[(int64_t)b * gamma + i] = nan;
        }
        wmul = w[tau];
    }
    ReqG r;
    r.flags = 0;
    r.L = L;
    r.tau = tau;
    r.mode = tau < L ? 0 : 1;
    r.wmul = wmul;
    r.lp2 = (float)lp2[tau];
    r.lq2 = tau < L ? (float)lq2[tau] : 0.0f;
    r.u2 = u2;
    req[b] = r;
}

// ---------------------------------------------------------------------------
// Correction / bonus weights.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float weight(float xp, float xq, int mode, float wmul, float lp2,
                                        float lq2, float c)
{
    const float pw = svk::fast_exp2(__builtin_fmaf(xp, c, -lp2));
    if (mode) return pw;
    const float qw = svk::fast_exp2(__builtin_fmaf(xq, c, -lq2));
    const float d = wmul * pw - qw;
    return d > 0.0f ? d : 0.0f;
}

// 8 consecutive elements starting at element e (16-byte aligned) of a row.
template <int ES>
__device__ __forceinline__ void load8(const char *row, int64_t e, float *x)
{
    const u32x4 *v = (const u32x4 *)(row + e * ES);
    if constexpr (ES == 2) {
        svk::widen<2>(__builtin_nontemporal_load(v), x);
    } else {
        svk::widen<4>(__builtin_nontemporal_load(v), x);
        svk::widen<4>(__builtin_nontemporal_load(v + 1), x + 4);
    }
}

// Sum of weights over elements [e0, e1) of the p / q rows, strided over the
// block (thread-local partial returned).
template <int PES, int QES>
__device__ float chunk_weight_sum(const char *prow, const char *qrow, int64_t e0, int64_t e1,
                                  int mode, float wmul, float lp2, float lq2, float c)
{
    float acc = 0.0f;
    const bool aligned = (((uintptr_t)(prow + e0 * PES)) & 15) == 0 &&
                         (mode || (((uintptr_t)(qrow + e0 * QES)) & 15) == 0);
    int64_t e_vec_end = e0;
    if (aligned) {
        const int64_t nunit = (e1 - e0) / 8;
        for (int64_t u = threadIdx.x; u < nunit; u += NT) {
            const int64_t e = e0 + u * 8;
            float xp[8], xq[8];
            load8<PES>(prow, e, xp);
            if (!mode) load8<QES>(qrow, e, xq);
#pragma unroll
            for (int k = 0; k < 8; ++k) acc += weight(xp[k], mode ? 0.0f : xq[k], mode, wmul, lp2, lq2, c);
        }
        e_vec_end = e0 + nunit * 8;
    }
    for (int64_t e = e_vec_end + threadIdx.x; e < e1; e += NT) {
        const float xp = svk::load_logit<PES>(prow, e);
        const float xq = mode ? 0.0f : svk::load_logit<QES>(qrow, e);
        acc += weight(xp, xq, mode, wmul, lp2, lq2, c);
    }
    return acc;
}

template <int PES, int QES>
__global__ __launch_bounds__(NT) void k_block_pass2(svh::VerifyArgs a, const ReqG *__restrict__ req,
                                                    const float *__restrict__ lp2g,
                                                    const float *__restrict__ lq2g,
                                                    const float *__restrict__ wrun, float *__restrict__ bm,
                                                    int nchr)
{
    __shared__ float red[NT / svk::kWave];
    const int gm1 = a.gamma - 1;
    const int64_t wg = blockIdx.x;
    const int c = (int)(wg % nchr);
    const int64_t bi = wg / nchr;
    const int b = (int)(bi / gm1);
    const int i = (int)(bi - (int64_t)b * gm1) + 1;   // 1..gamma-1
    const ReqG r = req[b];
    if (r.flags || i >= r.L) return;
    const int G1 = a.gamma + 1;
    const float w = wrun[(int64_t)b * G1 + i];
    const int64_t e0 = (int64_t)c * CHR;
    const int64_t e1 = e0 + CHR < a.V ? e0 + CHR : a.V;
    const char *prow = (const char *)a.p + ((int64_t)b * G1 + i) * a.V * PES;
    const char *qrow = (const char *)a.q + ((int64_t)b * a.gamma + i) * a.V * QES;
    const float acc = chunk_weight_sum<PES, QES>(prow, qrow, e0, e1, 0, w, lp2g[(int64_t)b * G1 + i],
                                                 lq2g[(int64_t)b * a.gamma + i], a.c);
    const float tot = svk::block_sum<NT>(acc, red);
    if (threadIdx.x == 0) bm[((int64_t)b * a.gamma + i) * nchr + c] = tot;
}

// Block pass 2 already summed the correction weights when 1 <= tau < L.
__device__ __forceinline__ bool sums_from_pass2(const svh::VerifyArgs &a, const ReqG &r)
{
    return a.block && r.mode == 0 && r.tau >= 1;
}

template <int PES, int QES>
__global__ __launch_bounds__(NT) void k_resid_sum(svh::VerifyArgs a, const ReqG *__restrict__ req,
                                                  float *__restrict__ csum, int nchr)
{
    __shared__ float red[NT / svk::kWave];
    const int64_t wg = blockIdx.x;
    const int b = (int)(wg / nchr);
    const int c = (int)(wg - (int64_t)b * nchr);
    const ReqG r = req[b];
    if (r.flags || sums_from_pass2(a, r)) return;
    const int G1 = a.gamma + 1;
    const char *prow = (const char *)a.p + ((int64_t)b * G1 + r.tau) * a.V * PES;
    const char *qrow = r.mode ? nullptr : (const char *)a.q + ((int64_t)b * a.gamma + r.tau) * a.V * QES;
    const int64_t e0 = (int64_t)c * CHR;
    const int64_t e1 = e0 + CHR < a.V ? e0 + CHR : a.V;
    const float acc = chunk_weight_sum<PES, QES>(prow, qrow, e0, e1, r.mode, r.wmul, r.lp2, r.lq2, a.c);
    const float tot = svk::block_sum<NT>(acc, red);
    if (threadIdx.x == 0) csum[(int64_t)b * nchr + c] = tot;
}

// ---------------------------------------------------------------------------
// Inverse-CDF selection, one workgroup per request.
// ---------------------------------------------------------------------------
struct SelectShared {
    double scan[NT];
    double cbase;          // cumulative weight before the chosen chunk
    int cstar;             // chosen chunk
    int clast;             // last chunk with positive weight
    int ybest;             // chosen token (min over threads)
    int ylast;             // last positive-weight token of the chunk
};

template <int PES, int QES>
__device__ int select_token(const svh::VerifyArgs &a, int mode, float wmul, float lp2, float lq2,
                            const float *sums, int nchr, const char *prow, const char *qrow, float u,
                            SelectShared &sh, double &Z_out)
{
    // chunk sums -> fp64 prefix (each thread owns a contiguous run of chunks)
    const int per = (nchr + NT - 1) / NT;
    const int k0 = threadIdx.x * per;
    const int k1 = k0 + per < nchr ? k0 + per : nchr;
    double loc = 0.0;
    for (int k = k0; k < k1; ++k) loc += (double)sums[k];
    double Z;
    const double excl = svk::block_exclusive_scan_d<NT>(loc, sh.scan, &Z);
    Z_out = Z;
    if (!(Z > 0.0)) return -1;
    const float tf = __fmul_rn(u, (float)Z);

    if (threadIdx.x == 0) {
        sh.cstar = 0x7FFFFFFF;
        sh.clast = -1;
        sh.ybest = 0x7FFFFFFF;
        sh.ylast = -1;
    }
    __syncthreads();
    {
        double run = excl;
        for (int k = k0; k < k1; ++k) {
            const float ck = sums[k];
            run += (double)ck;
            if (ck > 0.0f) {
                atomicMax(&sh.clast, k);
                if ((float)run > tf) {
                    atomicMin(&sh.cstar, k);
                    break;
                }
            }
        }
    }
    __syncthreads();
    const bool fallback = sh.cstar == 0x7FFFFFFF;
    const int cst = fallback ? sh.clast : sh.cstar;
    if (k0 <= cst && cst < k1) {
        double run = excl;
        for (int k = k0; k < cst; ++k) run += (double)sums[k];
        sh.cbase = run;
    }
    __syncthreads();

    // inside the chunk: each thread owns CHR / NT contiguous elements
    constexpr int PER = CHR / NT;
    const int64_t c0 = (int64_t)cst * CHR;
    const int64_t c1 = c0 + CHR < a.V ? c0 + CHR : a.V;
    const int64_t t0 = c0 + (int64_t)threadIdx.x * PER;
    float w[PER];
    double lsum = 0.0;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int64_t e = t0 + k;
        float wk = 0.0f;
        if (e < c1) {
            const float xp = svk::load_logit<PES>(prow, e);
            const float xq = mode ? 0.0f : svk::load_logit<QES>(qrow, e);
            wk = weight(xp, xq, mode, wmul, lp2, lq2, a.c);
        }
        w[k] = wk;
        lsum += (double)wk;
    }
    double dummy;
    const double texcl = svk::block_exclusive_scan_d<NT>(lsum, sh.scan, &dummy);
    int last_pos = -1;
#pragma unroll
    for (int k = 0; k < PER; ++k)
        if (w[k] > 0.0f) last_pos = (int)(t0 + k);
    if (last_pos >= 0) atomicMax(&sh.ylast, last_pos);
    if (!fallback) {
        double C = sh.cbase + texcl;
        for (int k = 0; k < PER; ++k) {
            C += (double)w[k];
            if (w[k] > 0.0f && (float)C > tf) {
                atomicMin(&sh.ybest, (int)(t0 + k));
                break;
            }
        }
    }
    __syncthreads();
    return sh.ybest != 0x7FFFFFFF ? sh.ybest : sh.ylast;
}

template <int PES, int QES>
__global__ __launch_bounds__(NT) void k_select(svh::VerifyArgs a, const ReqG *__restrict__ req,
                                               float *__restrict__ csum, const float *__restrict__ bm,
                                               int nchr, uint32_t *__restrict__ errword)
{
    __shared__ float red[NT / svk::kWave];
    __shared__ SelectShared sh;
    const int b = blockIdx.x;
    const ReqG r = req[b];
    if (r.flags) return;   // k_accept wrote the request's error outputs
    const int gamma = a.gamma;
    const int G1 = gamma + 1;
    const char *prow = (const char *)a.p + ((int64_t)b * G1 + r.tau) * a.V * PES;
    const char *qrow = r.mode ? nullptr : (const char *)a.q + ((int64_t)b * gamma + r.tau) * a.V * QES;
    float *own = csum + (int64_t)b * nchr;
    const float *sums = sums_from_pass2(a, r) ? bm + ((int64_t)b * gamma + r.tau) * nchr : own;

    uint32_t flags = 0;
    double Z = 0.0;
    int y = select_token<PES, QES>(a, r.mode, r.wmul, r.lp2, r.lq2, sums, nchr, prow, qrow, r.u2, sh, Z);
    if (y < 0 && r.mode == 0) {
        // residual mass rounded to zero (in exact arithmetic a rejection
        // implies p != q): draw from the p row instead
        flags |= SV_FLAG_RESID_ZERO;
        for (int k = 0; k < nchr; ++k) {
            const int64_t e0 = (int64_t)k * CHR;
            const int64_t e1 = e0 + CHR < a.V ? e0 + CHR : a.V;
            const float acc = chunk_weight_sum<PES, QES>(prow, nullptr, e0, e1, 1, 1.0f, r.lp2, 0.0f, a.c);
            const float tot = svk::block_sum<NT>(acc, red);
            if (threadIdx.x == 0) own[k] = tot;
            __syncthreads();
        }
        y = select_token<PES, QES>(a, 1, 1.0f, r.lp2, 0.0f, own, nchr, prow, nullptr, r.u2, sh, Z);
    }
    if (y < 0) flags |= SV_FLAG_BAD_ROW;   // unreachable for a valid row: p sums to 1
    if (threadIdx.x == 0) {
        const int64_t ob = (int64_t)b * G1;
        if (y >= 0) {
            for (int j = 0; j < G1; ++j)
                a.out_tokens[ob + j] = j < r.tau ? a.draft[(int64_t)b * gamma + j] : (j == r.tau ? y : -1);
            a.accepted_len[b] = r.tau;
        } else {
            for (int j = 0; j < G1; ++j) a.out_tokens[ob + j] = -1;
            a.accepted_len[b] = -1;
        }
        if (a.diag.flags) a.diag.flags[b] = flags;
        if (a.diag.resid_mass) a.diag.resid_mass[b] = (float)Z;
        if (flags) atomicOr(errword, flags);
    }
}

// ---------------------------------------------------------------------------
// Launch sequences.
// ---------------------------------------------------------------------------
template <int PES, int QES>
void launch_accept(sv_ctx *ctx, const svh::VerifyArgs &a, hipStream_t s, int stage)
{
    const int slot = svh::prof_begin(ctx, s, SV_KERNEL_ACCEPT);
    hipLaunchKernelGGL((k_accept<PES, QES>), dim3(a.B), dim3(svk::kWave), 0, s, a,
                       (const float2 *)ctx->ws.part, ctx->nch1, (const float *)ctx->ws.bm, ctx->nchr, stage,
                       (ReqG *)ctx->ws.req, ctx->ws.lp2, ctx->ws.lq2, ctx->ws.wrun, ctx->ws.errword);
    svh::prof_end(ctx, s, slot);
}

template <int PES, int QES>
void launch_sum_and_select(sv_ctx *ctx, const svh::VerifyArgs &a, hipStream_t s)
{
    const ReqG *req = (const ReqG *)ctx->ws.req;
    const int nchr = ctx->nchr;
    int slot = svh::prof_begin(ctx, s, SV_KERNEL_RESID);
    hipLaunchKernelGGL((k_resid_sum<PES, QES>), dim3((unsigned)((int64_t)a.B * nchr)), dim3(NT), 0, s, a, req,
                       ctx->ws.csum, nchr);
    svh::prof_end(ctx, s, slot);
    slot = svh::prof_begin(ctx, s, SV_KERNEL_SELECT);
    hipLaunchKernelGGL((k_select<PES, QES>), dim3(a.B), dim3(NT), 0, s, a, req, ctx->ws.csum,
                       (const float *)ctx->ws.bm, nchr, ctx->ws.errword);
    svh::prof_end(ctx, s, slot);
}

template <int PES, int QES>
hipError_t token_tail(sv_ctx *ctx, const svh::VerifyArgs &a, hipStream_t s)
{
    launch_accept<PES, QES>(ctx, a, s, STAGE_TOKEN);
    launch_sum_and_select<PES, QES>(ctx, a, s);
    return hipGetLastError();
}

template <int PES, int QES>
hipError_t block_tail(sv_ctx *ctx, const svh::VerifyArgs &a, hipStream_t s)
{
    launch_accept<PES, QES>(ctx, a, s, STAGE_BLOCK_PRE);
    if (a.gamma >= 2) {
        const int slot = svh::prof_begin(ctx, s, SV_KERNEL_BLOCK_PASS2);
        hipLaunchKernelGGL((k_block_pass2<PES, QES>), dim3((unsigned)((int64_t)a.B * (a.gamma - 1) * ctx->nchr)),
                           dim3(NT), 0, s, a, (const ReqG *)ctx->ws.req, (const float *)ctx->ws.lp2,
                           (const float *)ctx->ws.lq2, (const float *)ctx->ws.wrun, ctx->ws.bm, ctx->nchr);
        svh::prof_end(ctx, s, slot);
    }
    launch_accept<PES, QES>(ctx, a, s, STAGE_BLOCK_FINAL);
    launch_sum_and_select<PES, QES>(ctx, a, s);
    return hipGetLastError();
}

}  // namespace

namespace svh {

hipError_t launch_token_tail(sv_ctx *ctx, const VerifyArgs &a, hipStream_t s)
{
    if (a.B <= 0) return hipSuccess;
    if (a.p_esize == 2 && a.q_esize == 2) return token_tail<2, 2>(ctx, a, s);
    if (a.p_esize == 2) return token_tail<2, 4>(ctx, a, s);
    if (a.q_esize == 2) return token_tail<4, 2>(ctx, a, s);
    return token_tail<4, 4>(ctx, a, s);
}

hipError_t launch_block_tail(sv_ctx *ctx, const VerifyArgs &a, hipStream_t s)
{
    if (a.B <= 0) return hipSuccess;
    if (a.p_esize == 2 && a.q_esize == 2) return block_tail<2, 2>(ctx, a, s);
    if (a.p_esize == 2) return block_tail<2, 4>(ctx, a, s);
    if (a.q_esize == 2) return block_tail<4, 2>(ctx, a, s);
    return block_tail<4, 4>(ctx, a, s);
}

}  // namespace svh
