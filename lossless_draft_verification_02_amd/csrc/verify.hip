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
// Kernels:
//  k_block_pass2  grid (request, position i in 1..gamma-1, chunk): partial
//                 sums of max(w_i p_{i+1} - q_{i+1}, 0) over one chunk.
//  k_resid        grid (request, chunk): every workgroup evaluates its
//                 request (one wavefront: merge row statistics, gather the
//                 draft tokens' logits, draw uniforms, scan for tau), then sums
//                 the correction / bonus weights of its chunk; the last
//                 workgroup of the request to finish (device-scope counter)
//                 picks the chunk holding u*Z and scans inside it for the
//                 token (inverse CDF in ascending token id order).
#include "sv_device.h"
#include "sv_internal.h"

namespace {

using svk::u32x4;

constexpr int NT = svh::kResidThreads;
constexpr int CHR = svh::kChunkR;
constexpr int MAXG = svh::kMaxGamma;
constexpr double kLn2d = 0.69314718055994530942;

// ---------------------------------------------------------------------------
// Per-request evaluation, shared through LDS.
// ---------------------------------------------------------------------------
struct ReqState {
    uint32_t flags;
    int L;
    int tau;
    int mode;            // 0: residual weights (wmul * p - q), 1: bonus weights (p)
    float wmul;          // multiplier of p in the residual weights
    float lp2, lq2;      // log2-sum-exp2 of the chosen p and q rows
    float u2;            // correction / bonus uniform
    double lp2_all[MAXG + 1];   // log2-sum-exp2 of every verified p / q row
    double lq2_all[MAXG];
    float r_all[MAXG];   // uncapped p/q ratio of each draft token
    float w_all[MAXG + 1];
    float h_all[MAXG + 1];
};

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

// Wavefront 0 evaluates request b into st; other threads wait at the barrier
// that follows the call.
template <int PES, int QES>
__device__ void eval_request(const svh::VerifyArgs &a, const float2 *__restrict__ part, int nch1,
                             const float *__restrict__ bm, int nchr, int b, ReqState &st)
{
    if (threadIdx.x >= svk::kWave) return;
    const int lane = threadIdx.x;
    const int gamma = a.gamma;
    const int L = a.verify_len ? a.verify_len[b] : gamma;
    if (L < 0 || L > gamma) {
        if (lane == 0) {
            st.flags = SV_FLAG_BAD_VERIFY_LEN;
            st.L = L;
        }
        return;
    }
    const int64_t prow0 = (int64_t)b * (gamma + 1);
    const int64_t qrow0 = (int64_t)a.B * (gamma + 1) + (int64_t)b * gamma;

    // tokens first: a bad token is reported alone
    bool badtok = false;
    for (int j = lane; j < L; j += svk::kWave) {
        const int32_t x = a.draft[(int64_t)b * gamma + j];
        if (x < 0 || (int64_t)x >= a.V) badtok = true;
    }
    if (__ballot(badtok)) {
        if (lane == 0) {
            st.flags = SV_FLAG_BAD_TOKEN;
            st.L = L;
        }
        return;
    }
    bool badrow = false;
    for (int j = lane; j <= L; j += svk::kWave) st.lp2_all[j] = merge_row(part, prow0 + j, nch1, badrow);
    for (int j = lane; j < L; j += svk::kWave) st.lq2_all[j] = merge_row(part, qrow0 + j, nch1, badrow);
    if (__ballot(badrow)) {
        if (lane == 0) {
            st.flags = SV_FLAG_BAD_ROW;
            st.L = L;
        }
        return;
    }
    // ratios of the draft tokens, in log2 space
    for (int j = lane; j < L; j += svk::kWave) {
        const int32_t x = a.draft[(int64_t)b * gamma + j];
        const double xp = (double)svk::load_logit<PES>(a.p, (prow0 + j) * a.V + x) * (double)a.c;
        const double xq = (double)svk::load_logit<QES>(a.q, ((int64_t)b * gamma + j) * a.V + x) * (double)a.c;
        const float r = (float)exp2((xp - st.lp2_all[j]) - (xq - st.lq2_all[j]));
        st.r_all[j] = (r != r) ? 0.0f : r;
    }
    // only this wavefront runs here: order its LDS writes before lane 0 reads
    // them (a workgroup barrier would pair with the other waves' barriers)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (lane != 0) return;

    const float u2 = a.uniforms ? a.uniforms[(int64_t)b * (gamma + 1) + gamma]
                                : svk::philox_uniform(a.seed, a.offset, (uint32_t)b, 0u, 1u);
    int tau;
    float wmul = 1.0f;
    int mode;
    if (!a.block) {
        tau = L;
        for (int j = 0; j < L; ++j) {
            const float ratio = fminf(st.r_all[j], 1.0f);
            const float u = a.uniforms ? a.uniforms[(int64_t)b * (gamma + 1) + j]
                                       : svk::philox_uniform(a.seed, a.offset, (uint32_t)b,
                                                             (uint32_t)(j + 1), 0u);
            if (!(u < ratio)) {
                tau = j;
                break;
            }
        }
        mode = tau < L ? 0 : 1;
    } else {
        // running capped ratio; w_all[i] is w_i (w_0 = 1)
        st.w_all[0] = 1.0f;
        for (int i = 1; i <= L; ++i) {
            const float prev = st.w_all[i - 1];
            const float prod = prev == 0.0f ? 0.0f : prev * st.r_all[i - 1];
            st.w_all[i] = fminf(prod, 1.0f);
        }
        // thresholds; residual masses come from block pass 2
        for (int i = 1; i < L; ++i) {
            double m = 0.0;
            const float *bmi = bm + ((int64_t)b * gamma + i) * nchr;
            for (int k = 0; k < nchr; ++k) m += (double)bmi[k];
            const double den = m + 1.0 - (double)st.w_all[i];
            st.h_all[i] = den > 0.0 ? (float)(m / den) : 1.0f;
        }
        if (L >= 1) st.h_all[L] = st.w_all[L];
        tau = 0;
        for (int i = 1; i <= L; ++i) {
            const float eta = a.uniforms ? a.uniforms[(int64_t)b * (gamma + 1) + i - 1]
                                         : svk::philox_uniform(a.seed, a.offset, (uint32_t)b,
                                                               (uint32_t)i, 0u);
            if (eta < st.h_all[i]) tau = i;
        }
        mode = tau < L ? 0 : 1;
        wmul = st.w_all[tau];
    }
    st.flags = 0;
    st.L = L;
    st.tau = tau;
    st.mode = mode;
    st.wmul = wmul;
    st.lp2 = (float)st.lp2_all[tau];
    st.lq2 = tau < L ? (float)st.lq2_all[tau] : 0.0f;
    st.u2 = u2;
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
__global__ __launch_bounds__(NT) void k_block_pass2(svh::VerifyArgs a, const float2 *__restrict__ part,
                                                    int nch1, float *__restrict__ bm, int nchr)
{
    __shared__ ReqState st;
    __shared__ float red[NT / svk::kWave];
    const int gm1 = a.gamma - 1;
    const int64_t wg = blockIdx.x;
    const int c = (int)(wg % nchr);
    const int64_t bi = wg / nchr;
    const int b = (int)(bi / gm1);
    const int i = (int)(bi - (int64_t)b * gm1) + 1;   // 1..gamma-1
    const int L = a.verify_len ? a.verify_len[b] : a.gamma;
    if (L < 0 || L > a.gamma || i >= L) return;

    if (threadIdx.x == 0) st.flags = 0;
    __syncthreads();
    // w_i needs only the ratios; evaluate in token mode (no thresholds yet)
    svh::VerifyArgs ta = a;
    ta.block = false;
    ta.uniforms = nullptr;
    eval_request<PES, QES>(ta, part, nch1, nullptr, nchr, b, st);
    __syncthreads();
    if (st.flags) return;
    if (threadIdx.x == 0) {
        float w = 1.0f;
        for (int j = 1; j <= i; ++j) {
            const float prod = w == 0.0f ? 0.0f : w * st.r_all[j - 1];
            w = fminf(prod, 1.0f);
        }
        st.wmul = w;
    }
    __syncthreads();
    const int64_t e0 = (int64_t)c * CHR;
    const int64_t e1 = e0 + CHR < a.V ? e0 + CHR : a.V;
    const char *prow = (const char *)a.p + ((int64_t)b * (a.gamma + 1) + i) * a.V * PES;
    const char *qrow = (const char *)a.q + ((int64_t)b * a.gamma + i) * a.V * QES;
    const float acc = chunk_weight_sum<PES, QES>(prow, qrow, e0, e1, 0, st.wmul, (float)st.lp2_all[i],
                                                 (float)st.lq2_all[i], a.c);
    const float tot = svk::block_sum<NT>(acc, red);
    if (threadIdx.x == 0) bm[((int64_t)b * a.gamma + i) * nchr + c] = tot;
}

// ---------------------------------------------------------------------------
// Last-workgroup inverse-CDF selection.
// ---------------------------------------------------------------------------
struct SelectShared {
    double scan[NT];
    double cbase;          // cumulative weight before the chosen chunk
    int cstar;             // chosen chunk
    int clast;             // last chunk with positive weight
    int ybest;             // chosen token (min over threads)
    int ylast;             // last positive-weight token of the chunk
    double total;
};

template <int PES, int QES>
__device__ int select_token(const svh::VerifyArgs &a, const ReqState &st, int mode, float *csum_b,
                            int nchr, const char *prow, const char *qrow, float tf_u,
                            SelectShared &sh, double &Z_out)
{
    // chunk sums -> fp64 prefix (each thread owns a contiguous run of chunks)
    const int per = (nchr + NT - 1) / NT;
    const int k0 = threadIdx.x * per;
    const int k1 = k0 + per < nchr ? k0 + per : nchr;
    double loc = 0.0;
    for (int k = k0; k < k1; ++k) loc += (double)csum_b[k];
    double Z;
    const double excl = svk::block_exclusive_scan_d<NT>(loc, sh.scan, &Z);
    Z_out = Z;
    if (!(Z > 0.0)) return -1;
    const float Zf = (float)Z;
    const float tf = __fmul_rn(tf_u, Zf);

    if (threadIdx.x == 0) {
        sh.cstar = 0x7FFFFFFF;
        sh.clast = -1;
    }
    __syncthreads();
    {
        double run = excl;
        for (int k = k0; k < k1; ++k) {
            const float ck = csum_b[k];
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
        for (int k = k0; k < cst; ++k) run += (double)csum_b[k];
        sh.cbase = run;
    }
    if (threadIdx.x == 0) {
        sh.ybest = 0x7FFFFFFF;
        sh.ylast = -1;
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
            wk = weight(xp, xq, mode, st.wmul, st.lp2, st.lq2, a.c);
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
__global__ __launch_bounds__(NT) void k_resid(svh::VerifyArgs a, const float2 *__restrict__ part,
                                              int nch1, const float *__restrict__ bm,
                                              float *__restrict__ csum, int nchr,
                                              uint32_t *__restrict__ counter,
                                              uint32_t *__restrict__ errword)
{
    __shared__ ReqState st;
    __shared__ float red[NT / svk::kWave];
    __shared__ SelectShared sh;
    __shared__ int is_last;
    const int64_t wg = blockIdx.x;
    const int b = (int)(wg / nchr);
    const int c = (int)(wg - (int64_t)b * nchr);
    const int gamma = a.gamma;
    const int G1 = gamma + 1;

    if (threadIdx.x == 0) st.flags = 0;
    __syncthreads();
    eval_request<PES, QES>(a, part, nch1, bm, nchr, b, st);
    __syncthreads();

    if (st.flags) {
        if (c == 0) {
            for (int j = threadIdx.x; j < G1; j += NT) a.out_tokens[(int64_t)b * G1 + j] = -1;
            if (threadIdx.x == 0) {
                a.accepted_len[b] = -1;
                if (a.diag.flags) a.diag.flags[b] = st.flags;
                if (a.diag.resid_mass) a.diag.resid_mass[b] = __builtin_nanf("");
                atomicOr(errword, st.flags);
            }
            for (int j = threadIdx.x; j < gamma; j += NT) {
                if (a.diag.lse_q) a.diag.lse_q[(int64_t)b * gamma + j] = __builtin_nanf("");
                if (a.diag.ratio) a.diag.ratio[(int64_t)b * gamma + j] = __builtin_nanf("");
                if (a.diag.w) a.diag.w[(int64_t)b * gamma + j] = __builtin_nanf("");
                if (a.diag.h) a.diag.h[(int64_t)b * gamma + j] = __builtin_nanf("");
            }
            for (int j = threadIdx.x; j < G1; j += NT)
                if (a.diag.lse_p) a.diag.lse_p[(int64_t)b * G1 + j] = __builtin_nanf("");
        }
        return;
    }
    const int L = st.L;
    if (c == 0) {
        const float nan = __builtin_nanf("");
        for (int j = threadIdx.x; j < G1; j += NT)
            if (a.diag.lse_p) a.diag.lse_p[(int64_t)b * G1 + j] = j <= L ? (float)(st.lp2_all[j] * kLn2d) : nan;
        for (int j = threadIdx.x; j < gamma; j += NT) {
            if (a.diag.lse_q) a.diag.lse_q[(int64_t)b * gamma + j] = j < L ? (float)(st.lq2_all[j] * kLn2d) : nan;
            if (a.diag.ratio) a.diag.ratio[(int64_t)b * gamma + j] = j < L ? fminf(st.r_all[j], 1.0f) : nan;
            if (a.diag.w) a.diag.w[(int64_t)b * gamma + j] = (a.block && j < L) ? st.w_all[j + 1] : nan;
            if (a.diag.h) a.diag.h[(int64_t)b * gamma + j] = (a.block && j < L) ? st.h_all[j + 1] : nan;
        }
    }

    const int tau = st.tau;
    const char *prow = (const char *)a.p + ((int64_t)b * G1 + tau) * a.V * PES;
    const char *qrow = tau < L ? (const char *)a.q + ((int64_t)b * gamma + tau) * a.V * QES : nullptr;
    float *csum_b = csum + (int64_t)b * nchr;
    {
        const int64_t e0 = (int64_t)c * CHR;
        const int64_t e1 = e0 + CHR < a.V ? e0 + CHR : a.V;
        const float acc = chunk_weight_sum<PES, QES>(prow, qrow, e0, e1, st.mode, st.wmul, st.lp2,
                                                     st.lq2, a.c);
        const float tot = svk::block_sum<NT>(acc, red);
        if (threadIdx.x == 0) {
            csum_b[c] = tot;
            __threadfence();
            const uint32_t prev = atomicAdd(&counter[b], 1u);
            is_last = prev == (uint32_t)(nchr - 1);
        }
    }
    __syncthreads();
    if (!is_last) return;
    __threadfence();
    __syncthreads();

    // last workgroup of the request: choose the token
    uint32_t flags = 0;
    int mode = st.mode;
    double Z = 0.0;
    int y = select_token<PES, QES>(a, st, mode, csum_b, nchr, prow, qrow, st.u2, sh, Z);
    if (y < 0 && mode == 0) {
        // residual mass rounded to zero: draw from the p row instead
        flags |= SV_FLAG_RESID_ZERO;
        mode = 1;
        __syncthreads();
        if (threadIdx.x == 0) st.mode = 1;
        __syncthreads();
        for (int k = 0; k < nchr; ++k) {
            const int64_t e0 = (int64_t)k * CHR;
            const int64_t e1 = e0 + CHR < a.V ? e0 + CHR : a.V;
            const float acc = chunk_weight_sum<PES, QES>(prow, nullptr, e0, e1, 1, 1.0f, st.lp2, 0.0f, a.c);
            const float tot = svk::block_sum<NT>(acc, red);
            if (threadIdx.x == 0) csum_b[k] = tot;
            __syncthreads();
        }
        y = select_token<PES, QES>(a, st, mode, csum_b, nchr, prow, nullptr, st.u2, sh, Z);
    }
    if (y < 0) {
        flags |= SV_FLAG_BAD_ROW;   // unreachable for a valid row: p sums to 1
    }
    if (threadIdx.x == 0) {
        const int64_t ob = (int64_t)b * G1;
        if (y >= 0) {
            for (int j = 0; j < G1; ++j)
                a.out_tokens[ob + j] = j < tau ? a.draft[(int64_t)b * gamma + j] : (j == tau ? y : -1);
            a.accepted_len[b] = tau;
        } else {
            for (int j = 0; j < G1; ++j) a.out_tokens[ob + j] = -1;
            a.accepted_len[b] = -1;
        }
        if (a.diag.flags) a.diag.flags[b] = flags;
        if (a.diag.resid_mass) a.diag.resid_mass[b] = (float)Z;
        if (flags) atomicOr(errword, flags);
        counter[b] = 0u;
    }
}

template <int PES, int QES>
hipError_t launch_resid_typed(sv_ctx *ctx, const svh::VerifyArgs &a, hipStream_t s)
{
    const int64_t grid = (int64_t)a.B * ctx->nchr;
    hipLaunchKernelGGL((k_resid<PES, QES>), dim3((unsigned)grid), dim3(NT), 0, s, a, ctx->ws.part,
                       ctx->nch1, ctx->ws.bm, ctx->ws.csum, ctx->nchr, ctx->ws.counter,
                       ctx->ws.errword);
    return hipGetLastError();
}

template <int PES, int QES>
hipError_t launch_pass2_typed(sv_ctx *ctx, const svh::VerifyArgs &a, hipStream_t s)
{
    const int64_t grid = (int64_t)a.B * (a.gamma - 1) * ctx->nchr;
    hipLaunchKernelGGL((k_block_pass2<PES, QES>), dim3((unsigned)grid), dim3(NT), 0, s, a,
                       ctx->ws.part, ctx->nch1, ctx->ws.bm, ctx->nchr);
    return hipGetLastError();
}

}  // namespace

namespace svh {

hipError_t launch_resid(sv_ctx *ctx, const VerifyArgs &a, hipStream_t s)
{
    if (a.B <= 0) return hipSuccess;
    const int slot = prof_begin(ctx, s, SV_KERNEL_RESID);
    hipError_t e;
    if (a.p_esize == 2 && a.q_esize == 2) e = launch_resid_typed<2, 2>(ctx, a, s);
    else if (a.p_esize == 2) e = launch_resid_typed<2, 4>(ctx, a, s);
    else if (a.q_esize == 2) e = launch_resid_typed<4, 2>(ctx, a, s);
    else e = launch_resid_typed<4, 4>(ctx, a, s);
    prof_end(ctx, s, slot);
    return e;
}

hipError_t launch_block_pass2(sv_ctx *ctx, const VerifyArgs &a, hipStream_t s)
{
    if (a.B <= 0 || a.gamma < 2) return hipSuccess;
    const int slot = prof_begin(ctx, s, SV_KERNEL_BLOCK_PASS2);
    hipError_t e;
    if (a.p_esize == 2 && a.q_esize == 2) e = launch_pass2_typed<2, 2>(ctx, a, s);
    else if (a.p_esize == 2) e = launch_pass2_typed<2, 4>(ctx, a, s);
    else if (a.q_esize == 2) e = launch_pass2_typed<4, 2>(ctx, a, s);
    else e = launch_pass2_typed<4, 4>(ctx, a, s);
    prof_end(ctx, s, slot);
    return e;
}

}  // namespace svh
