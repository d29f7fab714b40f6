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
//  k_block_pass2  grid (request, position i, segment group): each wavefront
//                 sums max(w_i p_{i+1} - q_{i+1}, 0) over one segment of
//                 kSegR consecutive tokens.  Requests whose longest prefix
//                 already passes (eta_L < w_L, found by the pre stage) are
//                 skipped: tau = L for them whatever the other thresholds.
//  k_resid_sum    grid (request, segment group): segment sums of the
//                 correction / bonus weights of row tau+1 (skipped when
//                 block pass 2 already summed exactly those weights).
//  k_select       one workgroup per request: picks the segment holding u * Z
//                 from the fp64 prefix of the segment sums, then scans inside
//                 it, one 16-byte vector per thread, for the token (inverse CDF
//                 in ascending token id order).
#include "sv_device.h"
#include "sv_internal.h"
#include "sv_rowstats.h"

// The acceptance, fused-tail and selection kernels are latency-bound: one
// wavefront's path through them (a few thousand instructions, run once per
// request) sets their time, and its instruction fetches on a cold CU are a
// good part of it, so they are compiled for size (measured: the one-launch
// small call 14.1 -> 13.3 us, the others unchanged).
#define SV_LATENCY_KERNEL __attribute__((minsize))

namespace {

using svk::u32x4;

constexpr int NT = svh::kResidThreads;
constexpr int SEG = svh::kSegR;
constexpr int MAXG = svh::kMaxGamma;
constexpr double kLn2d = 0.69314718055994530942;

enum Stage { STAGE_TOKEN = 0, STAGE_BLOCK_PRE = 1, STAGE_BLOCK_FINAL = 2 };

// The q row of request b's correction draw (position tau + 1).
template <int QES>
__device__ __forceinline__ const char *correction_qrow(const svh::VerifyArgs &a, int b, int tau)
{
    return (const char *)a.q + ((int64_t)b * a.gamma + tau) * a.V * QES;
}

using svh::ReqG;

// log2 sum exp2 of a row from its chunk partials (fp64 result); flags a bad row.
// M = max m_k, S = sum s_k exp2(m_k - M) in chunk order.  A row of up to
// kMergeHeld chunks is loaded at once (one memory round trip); longer rows
// load kMergeBatch partials at a time (one round trip per batch and pass).
constexpr int kMergeBatch = 8;
constexpr int kMergeHeld = 16;
__device__ double merge_row(const float2 *__restrict__ part, int64_t row, int nch1, bool &bad)
{
    const float2 *pr = part + row * nch1;
    float M = svk::neg_inf();
    float S = 0.0f;
    if (nch1 <= kMergeHeld) {
        float2 v[kMergeHeld];
#pragma unroll
        for (int j = 0; j < kMergeHeld; ++j) v[j] = j < nch1 ? pr[j] : make_float2(svk::neg_inf(), 0.0f);
#pragma unroll
        for (int j = 0; j < kMergeHeld; ++j) M = fmaxf(M, v[j].x);
        if (M == svk::neg_inf()) {
#pragma unroll
            for (int j = 0; j < kMergeHeld; ++j) S += v[j].y;   // 0, or NaN for a NaN element
        } else {
#pragma unroll
            for (int j = 0; j < kMergeHeld; ++j)
                if (j < nch1) S += v[j].y * exp2f(v[j].x - M);
        }
    } else {
        float2 v[kMergeBatch];
        for (int k0 = 0; k0 < nch1; k0 += kMergeBatch) {
#pragma unroll
            for (int j = 0; j < kMergeBatch; ++j) v[j] = k0 + j < nch1 ? pr[k0 + j] : make_float2(svk::neg_inf(), 0.0f);
#pragma unroll
            for (int j = 0; j < kMergeBatch; ++j) M = fmaxf(M, v[j].x);
        }
        for (int k0 = 0; k0 < nch1; k0 += kMergeBatch) {
#pragma unroll
            for (int j = 0; j < kMergeBatch; ++j) v[j] = k0 + j < nch1 ? pr[k0 + j] : make_float2(svk::neg_inf(), 0.0f);
            if (M == svk::neg_inf()) {
#pragma unroll
                for (int j = 0; j < kMergeBatch; ++j) S += v[j].y;
            } else {
#pragma unroll
                for (int j = 0; j < kMergeBatch; ++j)
                    if (k0 + j < nch1) S += v[j].y * exp2f(v[j].x - M);
            }
        }
    }
    if (!(S > 0.0f) || M == svk::pos_inf() || S == svk::pos_inf()) bad = true;
    return (double)M + log2((double)S);
}

// Residual masses m_i = sum of the nseg segment sums of position i (i = 1 ..
// L-1) of one request, by one wavefront: lane l adds segments l, l + 64, ...
// of a position, then a fixed-order wavefront reduction; the loads of 8
// positions are issued together.  Lane i - 1 returns m_i.
__device__ double residual_masses(const float *__restrict__ bmr, int L, int nseg, int lane)
{
    constexpr int PB = 8;   // positions per batch
    double mine = 0.0;
    for (int i0 = 1; i0 < L; i0 += PB) {
        double acc[PB];
#pragma unroll
        for (int j = 0; j < PB; ++j) acc[j] = 0.0;
        for (int k0 = 0; k0 < nseg; k0 += svk::kWave) {
            float v[PB];
#pragma unroll
            for (int j = 0; j < PB; ++j)
                v[j] = (i0 + j < L && k0 + lane < nseg) ? bmr[(int64_t)(i0 + j) * nseg + k0 + lane] : 0.0f;
#pragma unroll
            for (int j = 0; j < PB; ++j) acc[j] += (double)v[j];
        }
#pragma unroll
        for (int j = 0; j < PB; ++j) {
            const double t = svk::wave_sum_d(acc[j]);
            if (lane == i0 + j - 1) mine = t;
        }
    }
    return mine;
}

// ---------------------------------------------------------------------------
// Per-request evaluation by one wavefront.
// ---------------------------------------------------------------------------
struct AcceptLDS {
    double lp2[MAXG + 1];   // log2-sum-exp2 of the verified p rows
    double lq2[MAXG];       // ... and q rows
    double rr[MAXG];        // uncapped p/q ratio of each draft token
    int32_t x[MAXG];        // the draft tokens
};

// Evaluates request b with the calling wavefront (threads 0..63 of the
// workgroup; no workgroup barrier inside) and stores the result in *out:
// merges the row statistics, gathers the draft tokens' logits, draws the
// uniforms and decides tau.  Writes the request's diagnostics, and its error
// outputs when it has a data error.  Lane j owns draft position j + 1 and p /
// q row j (gamma <= 64); every load that does not depend on the verify length
// is issued first, so the evaluation costs about two memory round trips.
template <int PES, int QES>
__device__ void accept_eval(const svh::VerifyArgs &a, const float2 *__restrict__ part, int nch1,
                            const float *__restrict__ bm, int nseg, int stage, int b, const ReqG *pre, ReqG *out,
                            float *__restrict__ lp2g, float *__restrict__ lq2g, double *__restrict__ wrun,
                            uint32_t *__restrict__ errword, AcceptLDS &s)
{
    double *lp2 = s.lp2;
    double *lq2 = s.lq2;
    double *rr = s.rr;
    const int lane = threadIdx.x;
    const int gamma = a.gamma;
    const int G1 = gamma + 1;
    const float nan = __builtin_nanf("");
    const int64_t prow0 = (int64_t)b * G1;
    const int64_t qrow0 = (int64_t)a.B * G1 + (int64_t)b * gamma;

    // ---- independent loads
    const int L = a.verify_len ? a.verify_len[b] : gamma;
    const bool has_tok = lane < gamma;
    const int32_t x = has_tok ? a.draft[(int64_t)b * gamma + lane] : 0;
    const bool x_ok = x >= 0 && (int64_t)x < a.V;
    const int32_t xs = x_ok ? x : 0;   // in-bounds address even for a bad id
    float gp = 0.0f, gq = 0.0f;
    if (has_tok) {
        gp = svk::load_logit<PES>(a.p, (prow0 + lane) * a.V + xs);
        gq = a.q_zx ? a.q_zx[(int64_t)b * gamma + lane]   // the sampler's logit of the drafted token
                    : svk::load_logit<QES>(a.q, ((int64_t)b * gamma + lane) * a.V + xs);
    }
    // row statistics of every row the request may verify (rows beyond the
    // verify length hold stale values and are not used)
    bool bad_p = false, bad_q = false, bad_p64 = false;
    const double lp = lane <= gamma ? merge_row(part, prow0 + lane, nch1, bad_p) : 0.0;
    double lq = 0.0;
    if (has_tok) {
        if (a.q_lse2) {   // the sampler's log2-sum-exp2 of the draft row
            const float l = a.q_lse2[(int64_t)b * gamma + lane];
            bad_q = !(l == l) || l == svk::pos_inf() || l == svk::neg_inf();
            lq = (double)l;
        } else {
            lq = merge_row(part, qrow0 + lane, nch1, bad_q);
        }
    }
    const double lp64 = (gamma == svk::kWave && lane == 0) ? merge_row(part, prow0 + svk::kWave, nch1, bad_p64) : 0.0;
    float u = 1.0f;
    if (has_tok && stage != STAGE_BLOCK_PRE)
        u = a.uniforms ? a.uniforms[(int64_t)b * G1 + lane]
                       : svk::philox_uniform(a.seed, a.offset, (uint32_t)b, (uint32_t)(lane + 1), 0u);
    // block thresholds: running ratio and residual mass of position lane + 1
    // (not needed when the pre stage already decided tau = L)
    const int tau_pre = stage == STAGE_BLOCK_FINAL ? pre->tau : -1;
    double wi = 1.0;
    double mi = 0.0;
    if (stage == STAGE_BLOCK_FINAL) {
        if (lane + 1 <= gamma) wi = wrun[(int64_t)b * G1 + lane + 1];
        if (tau_pre < 0 && L >= 2) mi = residual_masses(bm + (int64_t)b * gamma * nseg, L, nseg, lane);
    }

    // ---- checks: verify length, then tokens (reported alone), then rows
    uint32_t flags = 0;
    if (L < 0 || L > gamma) flags = SV_FLAG_BAD_VERIFY_LEN;
    if (!flags && __ballot(lane < L && !x_ok)) flags = SV_FLAG_BAD_TOKEN;
    if (!flags && __ballot((lane <= L && bad_p) || (lane < L && bad_q) || (L == svk::kWave && bad_p64)))
        flags = SV_FLAG_BAD_ROW;
    if (flags) {
        if (lane == 0) {
            ReqG r{};
            r.flags = flags;
            r.L = L;
            *out = r;
        }
        if (stage == STAGE_BLOCK_PRE) return;   // the final stage reports it
        for (int j = lane; j < G1; j += svk::kWave) {
            a.out_tokens[(int64_t)b * G1 + j] = -1;
            if (a.diag.lse_p) a.diag.lse_p[(int64_t)b * G1 + j] = nan;
        }
        for (int j = lane; j < G1; j += svk::kWave)
            if (a.diag.uniform) a.diag.uniform[(int64_t)b * G1 + j] = nan;
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

    // ratio of the lane's draft token, log2 space, fp64
    if (has_tok) s.x[lane] = x;
    if (lane <= gamma) lp2[lane] = lp;
    if (gamma == svk::kWave && lane == 0) lp2[svk::kWave] = lp64;
    if (has_tok) {
        lq2[lane] = lq;
        const double dp = (double)gp * (double)a.c - lp;
        const double dq = (double)gq * (double)a.c - lq;
        const double r = exp2(dp - dq);
        rr[lane] = (lane < L && r == r) ? r : 0.0;
    }
    // only this wavefront runs: order its LDS writes before other lanes read them
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    if (stage == STAGE_BLOCK_PRE) {
        for (int j = lane; j <= L; j += svk::kWave) lp2g[(int64_t)b * G1 + j] = (float)lp2[j];
        for (int j = lane; j < L; j += svk::kWave) lq2g[(int64_t)b * gamma + j] = (float)lq2[j];
        if (lane == 0) {
            // binary64 running product, as the thresholds built from it
            // are ill-conditioned where m_i + 1 - w_i is small
            double w = 1.0;
            wrun[(int64_t)b * G1] = w;
            for (int i = 1; i <= L; ++i) {
                const double prod = w == 0.0 ? 0.0 : w * rr[i - 1];   // 0 * inf := 0
                w = fmin(prod, 1.0);
                wrun[(int64_t)b * G1 + i] = w;
            }
            // tau is the largest passing prefix, so eta_L < h_L = w_L decides
            // tau = L whatever the other thresholds are: such a request needs
            // no residual masses (unless the caller asked for every h_i)
            int tau_early = -1;
            if (L >= 1 && !a.diag.h) {
                const float eta = a.uniforms ? a.uniforms[(int64_t)b * G1 + L - 1]
                                             : svk::philox_uniform(a.seed, a.offset, (uint32_t)b, (uint32_t)L, 0u);
                if (eta < (float)w) tau_early = L;
            }
            ReqG r{};
            r.flags = 0;
            r.L = L;
            r.tau = tau_early;
            *out = r;
        }
        return;
    }

    // diagnostics of the evaluated positions
    for (int j = lane; j < G1; j += svk::kWave)
        if (a.diag.lse_p) a.diag.lse_p[(int64_t)b * G1 + j] = j <= L ? (float)(lp2[j] * kLn2d) : nan;
    if (has_tok) {
        if (a.diag.lse_q) a.diag.lse_q[(int64_t)b * gamma + lane] = lane < L ? (float)(lq * kLn2d) : nan;
        if (a.diag.ratio) a.diag.ratio[(int64_t)b * gamma + lane] = lane < L ? (float)fmin(rr[lane], 1.0) : nan;
    }
    if (a.diag.uniform && has_tok) a.diag.uniform[(int64_t)b * G1 + lane] = lane < L ? u : nan;

    // lane j takes the decision at position j + 1
    const bool active = lane < L;
    int tau;
    float wmul = 1.0f;
    if (stage == STAGE_TOKEN) {
        // accept x_{j+1} iff u < min(1, ratio); tau = first rejection
        const uint64_t rej = __ballot(active && !(u < (float)fmin(rr[lane], 1.0)));
        tau = rej ? (int)__builtin_ctzll(rej) : L;
        if (has_tok) {
            if (a.diag.w) a.diag.w[(int64_t)b * gamma + lane] = nan;
            if (a.diag.h) a.diag.h[(int64_t)b * gamma + lane] = nan;
        }
    } else {
        // h_i = m_i / (m_i + 1 - w_i) for i < L, h_L = w_L
        const int i = lane + 1;
        float h = 0.0f;
        if (active) {
            if (i < L) {
                const double den = mi + 1.0 - wi;
                h = den > 0.0 ? (float)(mi / den) : 1.0f;
            } else {
                h = (float)wi;
            }
        }
        const uint64_t pass = __ballot(active && u < h);    // eta_i < h_i
        tau = pass ? 64 - (int)__builtin_clzll(pass) : 0;   // largest passing i
        if (tau_pre >= 0) tau = tau_pre;                     // decided by the pre stage (= L)
        if (has_tok) {
            if (a.diag.w) a.diag.w[(int64_t)b * gamma + lane] = active ? (float)wi : nan;
            if (a.diag.h) a.diag.h[(int64_t)b * gamma + lane] = active ? h : nan;
        }
        wmul = tau == 0 ? 1.0f : (float)__shfl(wi, tau - 1, svk::kWave);   // w_tau (w_0 = 1)
    }
    if (lane != 0) return;
    ReqG r;
    r.flags = 0;
    r.L = L;
    r.tau = tau;
    r.mode = tau < L ? 0 : 1;
    r.wmul = wmul;
    r.lp2 = (float)lp2[tau];
    r.lq2 = tau < L ? (float)lq2[tau] : 0.0f;
    r.u2 = a.uniforms ? a.uniforms[(int64_t)b * G1 + gamma]
                      : svk::philox_uniform(a.seed, a.offset, (uint32_t)b, 0u, 1u);
    if (a.diag.uniform) a.diag.uniform[(int64_t)b * G1 + gamma] = r.u2;
    *out = r;
}

template <int PES, int QES>
__global__ __launch_bounds__(svk::kWave)
SV_LATENCY_KERNEL void k_accept(
    svh::VerifyArgs a, const float2 *__restrict__ part, int nch1, const float *__restrict__ bm, int nseg,
    int stage, ReqG *__restrict__ req, float *__restrict__ lp2g, float *__restrict__ lq2g,
    double *__restrict__ wrun, uint32_t *__restrict__ errword)
{
    __shared__ AcceptLDS s;
    const int b = a.b0 + (int)blockIdx.x;
    accept_eval<PES, QES>(a, part, nch1, bm, nseg, stage, b, req + b, req + b, lp2g, lq2g, wrun, errword, s);
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

// Sum of the weights of tokens [s0, s1) (one segment, s1 - s0 <= SEG) by the
// calling wavefront; every lane returns the total.  A full aligned segment is
// read as 4 x 16-byte vectors per lane per row, all issued before any math.
template <int PES, int QES>
__device__ float segment_weight_sum(const char *prow, const char *qrow, int64_t s0, int64_t s1, int mode,
                                    float wmul, float lp2, float lq2, float c)
{
    const int lane = threadIdx.x & (svk::kWave - 1);
    const bool aligned = (((uintptr_t)(prow + s0 * PES)) & 15) == 0 &&
                         (mode || (((uintptr_t)(qrow + s0 * QES)) & 15) == 0);
    float acc = 0.0f;
    if (aligned && s1 - s0 == SEG) {
        constexpr int U = SEG / 8 / svk::kWave;   // 8-token units per lane
        float xp[U][8], xq[U][8];
#pragma unroll
        for (int k = 0; k < U; ++k) load8<PES>(prow, s0 + (int64_t)(lane + svk::kWave * k) * 8, xp[k]);
        if (!mode) {
#pragma unroll
            for (int k = 0; k < U; ++k) load8<QES>(qrow, s0 + (int64_t)(lane + svk::kWave * k) * 8, xq[k]);
#pragma unroll
            for (int k = 0; k < U; ++k)
#pragma unroll
                for (int j = 0; j < 8; ++j) acc += weight(xp[k][j], xq[k][j], 0, wmul, lp2, lq2, c);
        } else {
#pragma unroll
            for (int k = 0; k < U; ++k)
#pragma unroll
                for (int j = 0; j < 8; ++j) acc += weight(xp[k][j], 0.0f, 1, wmul, lp2, lq2, c);
        }
    } else {
        const int64_t nunit = aligned ? (s1 - s0) / 8 : 0;
        for (int64_t u = lane; u < nunit; u += svk::kWave) {
            float xp[8], xq[8];
            load8<PES>(prow, s0 + u * 8, xp);
            if (!mode) load8<QES>(qrow, s0 + u * 8, xq);
#pragma unroll
            for (int j = 0; j < 8; ++j) acc += weight(xp[j], mode ? 0.0f : xq[j], mode, wmul, lp2, lq2, c);
        }
        for (int64_t e = s0 + nunit * 8 + lane; e < s1; e += svk::kWave) {
            const float xp = svk::load_logit<PES>(prow, e);
            const float xq = mode ? 0.0f : svk::load_logit<QES>(qrow, e);
            acc += weight(xp, xq, mode, wmul, lp2, lq2, c);
        }
    }
    return svk::wave_sum(acc);
}

// Raw 16-byte vectors of the lane's share of one full, aligned segment of
// the correction / bonus rows: U units of 8 tokens per row.
template <int PES, int QES>
struct SegRaw {
    static constexpr int U = SEG / 8 / svk::kWave;
    u32x4 p[U][PES / 2];
    u32x4 q[U][QES / 2];
};

template <int PES, int QES>
__device__ __forceinline__ void seg_load(SegRaw<PES, QES> &r, const char *prow, const char *qrow, int64_t s0,
                                         int mode, int lane)
{
    constexpr int U = SegRaw<PES, QES>::U;
#pragma unroll
    for (int k = 0; k < U; ++k) {
        const int64_t e = s0 + (int64_t)(lane + svk::kWave * k) * 8;
        const u32x4 *vp = (const u32x4 *)(prow + e * PES);
#pragma unroll
        for (int h = 0; h < PES / 2; ++h) r.p[k][h] = __builtin_nontemporal_load(vp + h);
        if (!mode) {
            const u32x4 *vq = (const u32x4 *)(qrow + e * QES);
#pragma unroll
            for (int h = 0; h < QES / 2; ++h) r.q[k][h] = __builtin_nontemporal_load(vq + h);
        }
    }
}

template <int PES, int QES>
__device__ __forceinline__ float seg_reduce(const SegRaw<PES, QES> &r, int mode, float wmul, float lp2,
                                            float lq2, float c)
{
    constexpr int U = SegRaw<PES, QES>::U;
    float acc = 0.0f;
#pragma unroll
    for (int k = 0; k < U; ++k) {
        float xp[8], xq[8];
#pragma unroll
        for (int h = 0; h < PES / 2; ++h) svk::widen<PES>(r.p[k][h], xp + h * (16 / PES));
        if (!mode) {
#pragma unroll
            for (int h = 0; h < QES / 2; ++h) svk::widen<QES>(r.q[k][h], xq + h * (16 / QES));
#pragma unroll
            for (int j = 0; j < 8; ++j) acc += weight(xp[j], xq[j], 0, wmul, lp2, lq2, c);
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) acc += weight(xp[j], 0.0f, 1, wmul, lp2, lq2, c);
        }
    }
    return acc;
}

// Segment sums of the correction / bonus weights of rows prow / qrow into
// sums[kfirst, kend), by NW wavefronts of the workgroup (wavefront wid takes
// segments kfirst + wid, kfirst + wid + NW, ...; kend is at most the row's
// segment count).  Full segments of 16-byte aligned rows are
// software-pipelined (unless both rows are fp32, where the second buffer would
// spill): the next segment's vectors are requested before the current one is
// reduced, so two segments per wavefront are in flight.
template <int PES, int QES, int NW>
__device__ void segment_sums(const svh::VerifyArgs &a, const char *prow, const char *qrow, int mode, float wmul,
                             float lp2, float lq2, int kend, float *sums, int kfirst = 0)
{
    const int lane = threadIdx.x & (svk::kWave - 1), wid = threadIdx.x / svk::kWave;
    const bool aligned = (((uintptr_t)prow) & 15) == 0 && (mode || (((uintptr_t)qrow) & 15) == 0);
    const int nf = aligned ? (int)(a.V / SEG) : 0;
    const int nfull = nf < kend ? nf : kend;   // segments [kfirst, kend) only
    int k = kfirst + wid;
    if constexpr (PES == 4 && QES == 4) {
        // fp32 rows: a second register buffer does not fit; one segment at a time
        for (; k < nfull; k += NW) {
            SegRaw<PES, QES> cur;
            seg_load<PES, QES>(cur, prow, qrow, (int64_t)k * SEG, mode, lane);
            const float tot = svk::wave_sum(seg_reduce<PES, QES>(cur, mode, wmul, lp2, lq2, a.c));
            if (lane == 0) sums[k] = tot;
        }
    } else if (k < nfull) {
        SegRaw<PES, QES> cur, nxt;
        seg_load<PES, QES>(cur, prow, qrow, (int64_t)k * SEG, mode, lane);
        for (; k < nfull; k += NW) {
            const int kn = k + NW;
            if (kn < nfull) seg_load<PES, QES>(nxt, prow, qrow, (int64_t)kn * SEG, mode, lane);
            const float tot = svk::wave_sum(seg_reduce<PES, QES>(cur, mode, wmul, lp2, lq2, a.c));
            if (lane == 0) sums[k] = tot;
            if (kn < nfull) cur = nxt;
        }
    }
    // the partial last segment, or every segment of unaligned rows
    for (; k < kend; k += NW) {
        const int64_t s0 = (int64_t)k * SEG;
        const int64_t s1 = s0 + SEG < a.V ? s0 + SEG : a.V;
        const float tot = segment_weight_sum<PES, QES>(prow, qrow, s0, s1, mode, wmul, lp2, lq2, a.c);
        if (lane == 0) sums[k] = tot;
    }
}

constexpr int SPW = svh::kSegPerWG;   // segments (wavefronts) per workgroup

template <int PES, int QES>
__global__ __launch_bounds__(NT) void k_block_pass2(svh::VerifyArgs a, const ReqG *__restrict__ req,
                                                    const float *__restrict__ lp2g,
                                                    const float *__restrict__ lq2g,
                                                    const double *__restrict__ wrun, float *__restrict__ bm,
                                                    int nseg)
{
    const int nwg = (nseg + SPW - 1) / SPW;
    const int gm1 = a.gamma - 1;
    const int64_t wg = blockIdx.x;
    const int g = (int)(wg % nwg);
    const int64_t bi = wg / nwg;
    const int bl = (int)(bi / gm1);
    const int i = (int)(bi - (int64_t)bl * gm1) + 1;   // 1..gamma-1
    const int b = a.b0 + bl;
    const int sidx = g * SPW + (int)(threadIdx.x / svk::kWave);
    const ReqG r = req[b];
    if (r.flags || r.tau >= 0 || i >= r.L || sidx >= nseg) return;   // whole wavefronts leave together
    const int G1 = a.gamma + 1;
    const float w = (float)wrun[(int64_t)b * G1 + i];
    const int64_t s0 = (int64_t)sidx * SEG;
    const int64_t s1 = s0 + SEG < a.V ? s0 + SEG : a.V;
    const char *prow = (const char *)a.p + ((int64_t)b * G1 + i) * a.V * PES;
    const char *qrow = (const char *)a.q + ((int64_t)b * a.gamma + i) * a.V * QES;
    const float tot = segment_weight_sum<PES, QES>(prow, qrow, s0, s1, 0, w, lp2g[(int64_t)b * G1 + i],
                                                   lq2g[(int64_t)b * a.gamma + i], a.c);
    if ((threadIdx.x & (svk::kWave - 1)) == 0) bm[((int64_t)b * a.gamma + i) * nseg + sidx] = tot;
}

// Writes request b's outputs, one thread per output column: x_1..x_tau, the
// drawn token y, then -1 (all -1 and accepted_len -1 when y < 0).
__device__ __forceinline__ void write_outputs(const svh::VerifyArgs &a, int b, int tau, int y,
                                              const int32_t *x, uint32_t flags, double Z,
                                              uint32_t *__restrict__ errword, int nthreads)
{
    const int G1 = a.gamma + 1;
    const int64_t ob = (int64_t)b * G1;
    for (int j = threadIdx.x; j < G1; j += nthreads)
        a.out_tokens[ob + j] = y < 0 ? -1 : (j < tau ? x[j] : (j == tau ? y : -1));
    if (threadIdx.x == 0) {
        a.accepted_len[b] = y < 0 ? -1 : tau;
        if (a.diag.flags) a.diag.flags[b] = flags;
        if (a.diag.resid_mass) a.diag.resid_mass[b] = (float)Z;
        if (flags) atomicOr(errword, flags);
    }
}

// Block pass 2 already summed the correction weights when 1 <= tau < L.
__device__ __forceinline__ bool sums_from_pass2(const svh::VerifyArgs &a, const ReqG &r)
{
    return a.block && r.mode == 0 && r.tau >= 1;
}

template <int PES, int QES>
__global__ __launch_bounds__(NT) void k_resid_sum(svh::VerifyArgs a, const ReqG *__restrict__ req,
                                                  float *__restrict__ csum, int nseg)
{
    const int nwg = (nseg + SPW - 1) / SPW;
    const int64_t wg = blockIdx.x;
    const int bl = (int)(wg / nwg);
    const int g = (int)(wg - (int64_t)bl * nwg);
    const int b = a.b0 + bl;
    const ReqG r = req[b];
    if (r.flags || sums_from_pass2(a, r)) return;
    const int G1 = a.gamma + 1;
    const char *prow = (const char *)a.p + ((int64_t)b * G1 + r.tau) * a.V * PES;
    const char *qrow = r.mode ? nullptr : correction_qrow<QES>(a, b, r.tau);
    const int kfirst = g * SPW, kend = kfirst + SPW < nseg ? kfirst + SPW : nseg;
    segment_sums<PES, QES, SPW>(a, prow, qrow, r.mode, r.wmul, r.lp2, r.lq2, kend, csum + (int64_t)b * nseg,
                                kfirst);
}

// Token rule, split tail, acceptance and sums in one launch: grid (request,
// segment group); wavefront 0 of every workgroup evaluates its request (the
// same loads and arithmetic in each, so every workgroup reaches the same
// tau), then the workgroup's wavefronts sum their segments of the correction
// / bonus row.  The first workgroup of a request stores its state for the
// selection and writes its diagnostics; an error output is the same from
// every workgroup.
template <int PES, int QES>
__global__ __launch_bounds__(NT) void k_accept_sum(svh::VerifyArgs a, const float2 *__restrict__ part, int nch1,
                                                   ReqG *__restrict__ req, float *__restrict__ csum, int nseg,
                                                   uint32_t *__restrict__ errword)
{
    __shared__ AcceptLDS as;
    __shared__ ReqG r;
    const int nwg = (nseg + SPW - 1) / SPW;
    const int64_t wg = blockIdx.x;
    const int bl = (int)(wg / nwg);
    const int g = (int)(wg - (int64_t)bl * nwg);
    const int b = a.b0 + bl;
    if (threadIdx.x < svk::kWave) {
        svh::VerifyArgs av = a;
        if (g != 0) av.diag = sv_diag{};   // diagnostics once per request
        accept_eval<PES, QES>(av, part, nch1, nullptr, nseg, STAGE_TOKEN, b, nullptr, &r, nullptr, nullptr, nullptr,
                              errword, as);
    }
    __syncthreads();
    if (g == 0 && threadIdx.x == 0) req[b] = r;
    if (r.flags) return;
    const int G1 = a.gamma + 1;
    const char *prow = (const char *)a.p + ((int64_t)b * G1 + r.tau) * a.V * PES;
    const char *qrow = r.mode ? nullptr : correction_qrow<QES>(a, b, r.tau);
    const int kfirst = g * SPW, kend = kfirst + SPW < nseg ? kfirst + SPW : nseg;
    segment_sums<PES, QES, SPW>(a, prow, qrow, r.mode, r.wmul, r.lp2, r.lq2, kend, csum + (int64_t)b * nseg,
                                kfirst);
}

// ---------------------------------------------------------------------------
// Inverse-CDF selection.
// ---------------------------------------------------------------------------
// Inverse-CDF selection by one wavefront (no workgroup barrier): the segment
// sums give an fp64 wavefront prefix that picks the segment holding u * Z;
// lane l then owns tokens [32 l, 32 l + 32) of that segment and a second
// wavefront prefix finds the token.  Same decisions as select_token: the
// smallest token whose fp32 cumulative weight exceeds fp32(u * fp32(Z)), else
// the last positive-weight token.  Returns -1 when the weights sum to 0.
__device__ __forceinline__ int wave_min_i(int v)
{
#pragma unroll
    for (int o = svk::kWave / 2; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o, svk::kWave));
    return v;
}
__device__ __forceinline__ int wave_max_i(int v)
{
#pragma unroll
    for (int o = svk::kWave / 2; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, svk::kWave));
    return v;
}

template <int PES, int QES>
__device__ int select_token_wave(const svh::VerifyArgs &a, int mode, float wmul, float lp2, float lq2,
                                 const float *sums, int nseg, const char *prow, const char *qrow, float u,
                                 double &Z_out)
{
    constexpr int TPL = SEG / svk::kWave;   // tokens per lane inside the segment (32)
    static_assert(TPL % 8 == 0, "whole 8-token units per lane");
    const int lane = threadIdx.x & (svk::kWave - 1);
    const int per = (nseg + svk::kWave - 1) / svk::kWave;
    const int k0 = lane * per;
    const int k1 = k0 + per < nseg ? k0 + per : nseg;
    double loc = 0.0;
    for (int k = k0; k < k1; ++k) loc += (double)sums[k];
    const double incl = svk::wave_inclusive_scan_d(loc);
    const double excl = incl - loc;
    const double Z = __shfl(incl, svk::kWave - 1, svk::kWave);
    Z_out = Z;
    if (!(Z > 0.0)) return -1;
    const float tf = __fmul_rn(u, (float)Z);
    int first = 0x7FFFFFFF, lastpos = -1;
    {
        double run = excl;
        for (int k = k0; k < k1; ++k) {
            const float ck = sums[k];
            run += (double)ck;
            if (ck > 0.0f) {
                lastpos = k;
                if ((float)run > tf) {
                    first = k;
                    break;
                }
            }
        }
    }
    const int cstar = wave_min_i(first);
    const int clast = wave_max_i(lastpos);
    const bool fallback = cstar == 0x7FFFFFFF;
    const int cst = fallback ? clast : cstar;   // >= 0: Z > 0 needs a positive segment
    double before = excl;
    for (int k = k0; k < k1 && k < cst; ++k) before += (double)sums[k];
    const double cbase = __shfl(before, cst / per, svk::kWave);

    // inside the segment
    const int64_t s0 = (int64_t)cst * SEG;
    const int64_t s1 = s0 + SEG < a.V ? s0 + SEG : a.V;
    const int64_t t0 = s0 + (int64_t)lane * TPL;
    const bool aligned = (((uintptr_t)(prow + s0 * PES)) & 15) == 0 &&
                         (mode || (((uintptr_t)(qrow + s0 * QES)) & 15) == 0);
    float w[TPL];
    const bool vec_path = aligned && t0 + TPL <= s1;
    // the other lanes load DB tokens per batch; batches past every such
    // lane's tokens (a short segment leaves later batches, or whole lanes,
    // empty) are skipped by the whole wavefront
    constexpr int DB = 4;
    int nbatch;
    {
        const int64_t left = s1 - t0;
        const int mine = vec_path || left <= 0 ? 0 : (left < TPL ? (int)left : TPL);
        nbatch = wave_max_i((mine + DB - 1) / DB);
    }
    if (vec_path) {
        // every vector of the lane's 32 tokens is requested before any is
        // used: one memory round trip
        constexpr int U = TPL / 8;
        u32x4 rp[U][PES / 2], rq[U][QES / 2];
#pragma unroll
        for (int g = 0; g < U; ++g) {
            const u32x4 *vp = (const u32x4 *)(prow + (t0 + 8 * g) * PES);
#pragma unroll
            for (int h = 0; h < PES / 2; ++h) rp[g][h] = __builtin_nontemporal_load(vp + h);
        }
        if (!mode) {
#pragma unroll
            for (int g = 0; g < U; ++g) {
                const u32x4 *vq = (const u32x4 *)(qrow + (t0 + 8 * g) * QES);
#pragma unroll
                for (int h = 0; h < QES / 2; ++h) rq[g][h] = __builtin_nontemporal_load(vq + h);
            }
        }
#pragma unroll
        for (int g = 0; g < U; ++g) {
            float xp[8], xq[8];
#pragma unroll
            for (int h = 0; h < PES / 2; ++h) svk::widen<PES>(rp[g][h], xp + h * (16 / PES));
            if (!mode) {
#pragma unroll
                for (int h = 0; h < QES / 2; ++h) svk::widen<QES>(rq[g][h], xq + h * (16 / QES));
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) w[8 * g + j] = weight(xp[j], mode ? 0.0f : xq[j], mode, wmul, lp2, lq2, a.c);
        }
    } else {
        // a partial or unaligned segment: DB elements at a time, each batch
        // requested before it is weighed (past the segment's end, an in-row
        // index whose weight is discarded), addressed by 32-bit offsets from
        // the segment start
        const int ts = (int)(t0 - s0), ns = (int)(s1 - s0);   // within the segment (< SEG)
#pragma unroll
        for (int g = 0; g < TPL / DB; ++g) {
            if (g >= nbatch) {   // wavefront-uniform: no lane has tokens left
#pragma unroll
                for (int j = 0; j < DB; ++j) w[DB * g + j] = 0.0f;
                continue;
            }
            float xp[DB], xq[DB];
#pragma unroll
            for (int j = 0; j < DB; ++j) {
                const int o = ts + DB * g + j;
                xp[j] = svk::load_logit<PES>(prow, s0 + (o < ns ? o : 0));
            }
            if (!mode) {
#pragma unroll
                for (int j = 0; j < DB; ++j) {
                    const int o = ts + DB * g + j;
                    xq[j] = svk::load_logit<QES>(qrow, s0 + (o < ns ? o : 0));
                }
            }
#pragma unroll
            for (int j = 0; j < DB; ++j)
                w[DB * g + j] = ts + DB * g + j < ns ? weight(xp[j], mode ? 0.0f : xq[j], mode, wmul, lp2, lq2, a.c)
                                                     : 0.0f;
            __builtin_amdgcn_sched_barrier(0);   // one batch of loads live at a time
        }
    }
    double lsum = 0.0;
#pragma unroll
    for (int j = 0; j < TPL; ++j) lsum += (double)w[j];
    const double tincl = svk::wave_inclusive_scan_d(lsum);
    int yl = -1, yb = 0x7FFFFFFF;
#pragma unroll
    for (int j = 0; j < TPL; ++j)
        if (w[j] > 0.0f) yl = (int)(t0 + j);
    if (!fallback) {
        double C = cbase + (tincl - lsum);
#pragma unroll
        for (int j = 0; j < TPL; ++j) {
            C += (double)w[j];
            if (yb == 0x7FFFFFFF && w[j] > 0.0f && (float)C > tf) yb = (int)(t0 + j);
        }
    }
    const int ybest = wave_min_i(yb);
    const int ylast = wave_max_i(yl);
    return ybest != 0x7FFFFFFF ? ybest : ylast;
}

// Split tail, selection: one wavefront per request draws the correction /
// bonus token from the segment sums (k_resid_sum's or block pass 2's) with
// the fused tail's wavefront draw.
template <int PES, int QES>
__global__ __launch_bounds__(svk::kWave)
SV_LATENCY_KERNEL void k_select(
    svh::VerifyArgs a, const ReqG *__restrict__ req, float *__restrict__ csum, const float *__restrict__ bm,
    int nseg, uint32_t *__restrict__ errword)
{
    __shared__ int32_t xs[MAXG];
    const int b = a.b0 + (int)blockIdx.x;
    const ReqG r = req[b];
    if (r.flags) return;   // k_accept wrote the request's error outputs
    const int gamma = a.gamma;
    const int G1 = gamma + 1;
    if ((int)threadIdx.x < r.tau) xs[threadIdx.x] = a.draft[(int64_t)b * gamma + threadIdx.x];
    const char *prow = (const char *)a.p + ((int64_t)b * G1 + r.tau) * a.V * PES;
    const char *qrow = r.mode ? nullptr : correction_qrow<QES>(a, b, r.tau);
    float *own = csum + (int64_t)b * nseg;
    const float *sums = sums_from_pass2(a, r) ? bm + ((int64_t)b * gamma + r.tau) * nseg : own;

    uint32_t flags = 0;
    double Z = 0.0;
    int y = select_token_wave<PES, QES>(a, r.mode, r.wmul, r.lp2, r.lq2, sums, nseg, prow, qrow, r.u2, Z);
    if (y < 0 && r.mode == 0) {
        // residual mass rounded to zero (in exact arithmetic a rejection
        // implies p != q): draw from the p row instead
        flags |= SV_FLAG_RESID_ZERO;
        segment_sums<PES, QES, 1>(a, prow, nullptr, 1, 1.0f, r.lp2, 0.0f, nseg, own);
        // lane 0 wrote the sums the whole wavefront reads next
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        y = select_token_wave<PES, QES>(a, 1, 1.0f, r.lp2, 0.0f, own, nseg, prow, nullptr, r.u2, Z);
    }
    if (y < 0) flags |= SV_FLAG_BAD_ROW;   // unreachable for a valid row: p sums to 1
    __syncthreads();   // xs written above
    write_outputs(a, b, r.tau, y, xs, flags, Z, errword, svk::kWave);
}

// ---------------------------------------------------------------------------
// Fused tail: one workgroup of NTT threads per request evaluates the request
// (wavefront 0), sums the correction / bonus weights of row tau+1 segment by
// segment into LDS (all wavefronts) and selects the token, with no
// communication between workgroups.  Used when the segment sums fit in LDS.
// ---------------------------------------------------------------------------
constexpr int NTT_WIDE = 1024;      // one workgroup per CU when requests <= CUs
constexpr int NTT_NARROW = 512;     // two per CU otherwise (<= 128 VGPRs either way)
constexpr int kTailMaxSeg = svh::kTailMaxSeg;   // LDS segment sums: V <= 8.4M tokens
#ifndef SV_FUSED_TAIL
#define SV_FUSED_TAIL 1             // 0: always the accept / sum / select kernels
#endif

// Small problems (rows of one chunk, few rows per request): the request's
// own workgroup computes the statistics of the rows it verifies before the
// tail runs -- wavefront w takes rows w, w + NW, ... (p rows 0..L, then q rows
// 0..L-1), each streamed once with the row-statistics pass's per-thread
// arithmetic and merged across the wavefront -- so a call is one launch.
// The pairs go to the same place the row-statistics pass puts them
// (nch1 == 1); the barrier after makes them visible to wavefront 0.
template <int PES, int QES, int NW>
__device__ void small_rowstats(const svh::VerifyArgs &a, int b, float2 *__restrict__ part)
{
    const int lane = threadIdx.x & (svk::kWave - 1), wid = threadIdx.x / svk::kWave;
    const int L = a.verify_len ? a.verify_len[b] : a.gamma;
    if (L < 0 || L > a.gamma) return;   // flagged by the acceptance
    const int np = a.gamma + 1, nq = a.gamma;
    for (int r = wid; r < 2 * L + 1; r += NW) {
        const bool is_p = r <= L;
        const int i = is_p ? r : r - (L + 1);
        svk::MS t;
        int64_t grow;
        if (is_p) {
            grow = (int64_t)b * np + i;
            t = svk::thread_stats<PES, 8, svk::kWave>((const char *)a.p + grow * a.V * PES, 0, a.V, a.c, true, lane);
        } else {
            const int64_t qr = (int64_t)b * nq + i;
            grow = (int64_t)a.B * np + qr;
            t = svk::thread_stats<QES, 8, svk::kWave>((const char *)a.q + qr * a.V * QES, 0, a.V, a.c, true, lane);
        }
        t = svk::wave_merge(t);
        if (lane == 0) part[grow] = make_float2(t.m, t.s);
    }
}

template <int PES, int QES, int NTT, bool SMALL>
__global__ __launch_bounds__(NTT, 4)
SV_LATENCY_KERNEL void k_tail(
    svh::VerifyArgs a, float2 *__restrict__ part, int nch1, int nseg, uint32_t *__restrict__ errword)
{
    __shared__ AcceptLDS as;
    __shared__ ReqG r;
    __shared__ float segsum[kTailMaxSeg];
    __shared__ int ybest;   // the draw's token (wavefront 0)
    const int b = a.b0 + (int)blockIdx.x;
    if constexpr (SMALL) {   // token verification of a small problem: its row statistics first
        small_rowstats<PES, QES, NTT / svk::kWave>(a, b, part);
        __syncthreads();
    }
    if (threadIdx.x < svk::kWave) {
        accept_eval<PES, QES>(a, part, nch1, nullptr, nseg, STAGE_TOKEN, b, nullptr, &r, nullptr, nullptr, nullptr,
                              errword, as);
    }
    __syncthreads();
    if (r.flags) return;   // the request's error outputs are written
    const int gamma = a.gamma;
    const int G1 = gamma + 1;
    const int lane = threadIdx.x & (svk::kWave - 1), wid = threadIdx.x / svk::kWave;
    const char *prow = (const char *)a.p + ((int64_t)b * G1 + r.tau) * a.V * PES;
    const char *qrow = r.mode ? nullptr : correction_qrow<QES>(a, b, r.tau);

    const float *sums = segsum;
    segment_sums<PES, QES, NTT / svk::kWave>(a, prow, qrow, r.mode, r.wmul, r.lp2, r.lq2, nseg, segsum);
    __syncthreads();
    // the draw: wavefront 0 alone
    uint32_t flags = 0;
    double Z = 0.0;
    int y = 0;
    if (wid == 0) {
        y = select_token_wave<PES, QES>(a, r.mode, r.wmul, r.lp2, r.lq2, sums, nseg, prow, qrow, r.u2, Z);
        if (lane == 0) ybest = y;
    }
    __syncthreads();
    if (ybest < 0 && r.mode == 0) {
        // residual mass rounded to zero (in exact arithmetic a rejection
        // implies p != q): draw from the p row instead
        flags |= SV_FLAG_RESID_ZERO;
        for (int k = wid; k < nseg; k += NTT / svk::kWave) {
            const int64_t s0 = (int64_t)k * SEG;
            const int64_t s1 = s0 + SEG < a.V ? s0 + SEG : a.V;
            const float tot = segment_weight_sum<PES, QES>(prow, nullptr, s0, s1, 1, 1.0f, r.lp2, 0.0f, a.c);
            if (lane == 0) segsum[k] = tot;
        }
        __syncthreads();
        if (wid == 0) y = select_token_wave<PES, QES>(a, 1, 1.0f, r.lp2, 0.0f, segsum, nseg, prow, nullptr, r.u2, Z);
    }
    if (wid != 0) return;
    if (y < 0) flags |= SV_FLAG_BAD_ROW;   // unreachable for a valid row: p sums to 1
    write_outputs(a, b, r.tau, y, as.x, flags, Z, errword, svk::kWave);
}

// ---------------------------------------------------------------------------
// Launch sequences.
// ---------------------------------------------------------------------------
template <int PES, int QES>
void launch_accept(sv_ctx *ctx, const svh::VerifyArgs &a, hipStream_t s, int stage)
{
    const int slot = svh::prof_begin(ctx, s, SV_KERNEL_ACCEPT);
    hipLaunchKernelGGL((k_accept<PES, QES>), dim3(a.nb), dim3(svk::kWave), 0, s, a,
                       (const float2 *)ctx->ws.part, ctx->nch1, (const float *)ctx->ws.bm, ctx->nseg, stage,
                       (ReqG *)ctx->ws.req, ctx->ws.lp2, ctx->ws.lq2, ctx->ws.wrun, ctx->ws.errword);
    svh::prof_end(ctx, s, slot);
}

template <int PES, int QES>
void launch_sum_and_select(sv_ctx *ctx, const svh::VerifyArgs &a, hipStream_t s)
{
    const ReqG *req = (const ReqG *)ctx->ws.req;
    const int nseg = ctx->nseg;
    const int64_t nwg = (nseg + SPW - 1) / SPW;
    int slot = svh::prof_begin(ctx, s, SV_KERNEL_RESID);
    hipLaunchKernelGGL((k_resid_sum<PES, QES>), dim3((unsigned)((int64_t)a.nb * nwg)), dim3(NT), 0, s, a, req,
                       ctx->ws.csum, nseg);
    svh::prof_end(ctx, s, slot);
    slot = svh::prof_begin(ctx, s, SV_KERNEL_SELECT);
    hipLaunchKernelGGL((k_select<PES, QES>), dim3(a.nb), dim3(svk::kWave), 0, s, a, req, ctx->ws.csum,
                       (const float *)ctx->ws.bm, nseg, ctx->ws.errword);
    svh::prof_end(ctx, s, slot);
}

// The fused tail (token rule): small = 1 adds the row statistics (one launch
// for a small problem).
template <int PES, int QES>
void launch_fused_tail(sv_ctx *ctx, const svh::VerifyArgs &a, hipStream_t s, int small = 0)
{
    const int slot = svh::prof_begin(ctx, s, SV_KERNEL_TAIL);
    if (small)
        hipLaunchKernelGGL((k_tail<PES, QES, NTT_WIDE, true>), dim3(a.nb), dim3(NTT_WIDE), 0, s, a, ctx->ws.part,
                           ctx->nch1, ctx->nseg, ctx->ws.errword);
    else if (a.nb <= ctx->num_cu)
        hipLaunchKernelGGL((k_tail<PES, QES, NTT_WIDE, false>), dim3(a.nb), dim3(NTT_WIDE), 0, s, a, ctx->ws.part,
                           ctx->nch1, ctx->nseg, ctx->ws.errword);
    else
        hipLaunchKernelGGL((k_tail<PES, QES, NTT_NARROW, false>), dim3(a.nb), dim3(NTT_NARROW), 0, s, a,
                           ctx->ws.part, ctx->nch1, ctx->nseg, ctx->ws.errword);
    svh::prof_end(ctx, s, slot);
}

// One launch for token verification of a small problem: rows of a single
// row-statistics chunk, at most kSmallRowsPerWave rows per wavefront of the
// 1024-thread tail, and not more requests than two per CU (beyond that the
// row-statistics pass spreads the rows better).
constexpr int kSmallRowsPerWave = 4;
inline bool small_fits(const sv_ctx *ctx, const svh::VerifyArgs &a)
{
    return SV_FUSED_TAIL && ctx->nch1 == 1 && !a.q_lse2 && a.np_rows == 0 && !a.block &&
           2 * a.gamma + 1 <= kSmallRowsPerWave * (NTT_WIDE / svk::kWave) && a.nb <= 2 * ctx->num_cu;
}

// The fused tail puts each request's segment sums on one CU, which streams
// a 2-row pass at its share of the bandwidth; a batch that would leave most
// CUs idle spreads them over workgroups per segment group instead
// (k_resid_sum), at the price of two more launches.
inline bool fused_tail_fits(const sv_ctx *ctx, const svh::VerifyArgs &a)
{
    if (!SV_FUSED_TAIL || ctx->nseg > kTailMaxSeg) return false;
    return !(4 * (int64_t)a.nb <= ctx->num_cu && ctx->nseg >= 16);
}

template <int PES, int QES>
hipError_t token_single(sv_ctx *ctx, const svh::VerifyArgs &a, hipStream_t s)
{
    launch_fused_tail<PES, QES>(ctx, a, s, 1);
    return hipGetLastError();
}

template <int PES, int QES>
hipError_t token_tail(sv_ctx *ctx, const svh::VerifyArgs &a, hipStream_t s)
{
    if (fused_tail_fits(ctx, a)) {
        launch_fused_tail<PES, QES>(ctx, a, s);
    } else {
        const int nseg = ctx->nseg;
        const int64_t nwg = (nseg + SPW - 1) / SPW;
        int slot = svh::prof_begin(ctx, s, SV_KERNEL_RESID);
        hipLaunchKernelGGL((k_accept_sum<PES, QES>), dim3((unsigned)((int64_t)a.nb * nwg)), dim3(NT), 0, s, a,
                           (const float2 *)ctx->ws.part, ctx->nch1, (ReqG *)ctx->ws.req, ctx->ws.csum, nseg,
                           ctx->ws.errword);
        svh::prof_end(ctx, s, slot);
        slot = svh::prof_begin(ctx, s, SV_KERNEL_SELECT);
        hipLaunchKernelGGL((k_select<PES, QES>), dim3(a.nb), dim3(svk::kWave), 0, s, a, (const ReqG *)ctx->ws.req,
                           ctx->ws.csum, (const float *)ctx->ws.bm, nseg, ctx->ws.errword);
        svh::prof_end(ctx, s, slot);
    }
    return hipGetLastError();
}

template <int PES, int QES>
hipError_t block_tail(sv_ctx *ctx, const svh::VerifyArgs &a, hipStream_t s)
{
    launch_accept<PES, QES>(ctx, a, s, STAGE_BLOCK_PRE);
    if (a.gamma >= 2) {
        const int slot = svh::prof_begin(ctx, s, SV_KERNEL_BLOCK_PASS2);
        const int64_t nwg = (ctx->nseg + SPW - 1) / SPW;
        hipLaunchKernelGGL((k_block_pass2<PES, QES>), dim3((unsigned)((int64_t)a.nb * (a.gamma - 1) * nwg)),
                           dim3(NT), 0, s, a, (const ReqG *)ctx->ws.req, (const float *)ctx->ws.lp2,
                           (const float *)ctx->ws.lq2, (const double *)ctx->ws.wrun, ctx->ws.bm, ctx->nseg);
        svh::prof_end(ctx, s, slot);
    }
    // the final stage, then the correction / bonus sums over many workgroups
    // per request (most requests' sums come from pass 2; the rest stream a
    // row or two, which one workgroup per request would do at one CU's
    // rate), then the selection
    launch_accept<PES, QES>(ctx, a, s, STAGE_BLOCK_FINAL);
    launch_sum_and_select<PES, QES>(ctx, a, s);
    return hipGetLastError();
}

template <int PES>
hipError_t markov_verify_tail(sv_ctx *ctx, const svh::VerifyArgs &a, const svh::MarkovArgs &m, hipStream_t s)
{
    launch_accept<PES, 4>(ctx, a, s, STAGE_TOKEN);
    return svh::launch_markov_resid(ctx, m, a, (const ReqG *)ctx->ws.req, s);
}

// ---------------------------------------------------------------------------
// Tree verification ("Speculative Decoding: The Same Distribution, Twice as
// Fast", section 7: several alternative continuations arranged as a tree and
// checked in one pass), by recursive rejection: the children of a node were
// drawn independently from the draft q at that node; each child is accepted
// with probability min(1, r(x)/q(x)) for the current residual r, which is p
// at the node and after each rejection becomes max(r - q, 0) normalised; if
// every child is rejected the token is drawn from r, at a leaf from p.
// After j >= 1 rejections r is proportional to max(p - A_j q, 0), A_1 = 1,
// A_{j+1} = A_j (1 + Z_j) with Z_j the mass of max(p / A_j - q, 0): the
// residual stays the correction weights max(wmul p - q, 0) of the token
// sampler with wmul = 1 / A_j, and each rejection costs one pass over the
// node's p and q rows for the next Z.  The first child takes the token rule's
// log-space ratio, so a chain-shaped tree is token verification.
//
// One workgroup per request.  Wavefront 0 walks the tree: its lanes first
// gather every node's token logits under the node's parent rows (one memory
// round trip for the whole tree, independent of the decisions); lane 0 then
// decides.
// Between decisions that need a residual mass, and for the final draw, all
// wavefronts sum the current weights over the node's rows into LDS segment
// sums (the fused tail's segment sums and wavefront draw).
// ---------------------------------------------------------------------------
struct TreeLDS {
    double lp[MAXG + 1];        // log2-sum-exp2 of every p row (node order)
    double lq[MAXG + 1];        // ... of every q row (order of the nodes with children)
    float zp[MAXG + 1];         // node m's token logit in its parent's p row ...
    float zq[MAXG + 1];         // ... and q row (gathered when the parent is reached)
    float u[MAXG + 1];          // node m's acceptance uniform
    int32_t x[MAXG];            // token of node m at x[m - 1]
    int32_t path_x[MAXG], path_n[MAXG];
    double zr;                  // mass of the current residual weights
    double wmul;                // residual weights max(wmul p - q, 0)
    int node, child, depth, act, mode, first, resid_p;
    uint32_t flags;
};
enum { TREE_PASS = 0, TREE_DRAW = 1, TREE_DONE = 2 };

__device__ __forceinline__ int64_t tree_prow(const svh::TreeTopo &t, int b, int n) { return (int64_t)b * (t.N + 1) + n; }
__device__ __forceinline__ int64_t tree_qrow(const svh::TreeTopo &t, int b, int n) { return (int64_t)b * t.NQ + t.qrow[n]; }

// Wavefront 0, lane 0: decisions at st.node from st.child on, until a pass
// or the draw is needed (st.act says which).
__device__ void tree_decide(const svh::VerifyArgs &a, const svh::TreeTopo &t, int b, TreeLDS &st, bool writer)
{
    for (;;) {
    const int node = st.node;
    if (t.first_child[node] < 0) {   // a leaf: the bonus token from p
        st.mode = 1;
        st.wmul = 1.0;
        st.act = TREE_DRAW;
        return;
    }
    const double lp = st.lp[node], lq = st.lq[t.qrow[node]];
    const float lp2 = (float)lp, lq2 = (float)lq;
    {
        const int c = st.child;
        const float zp = st.zp[c], zq = st.zq[c];
        float ratio;
        if (st.first) {   // the token rule's ratio, log2 space in fp64
            const double dp = (double)zp * (double)a.c - lp;
            const double dq = (double)zq * (double)a.c - lq;
            const float r = (float)exp2(dp - dq);
            ratio = r == r ? fminf(r, 1.0f) : 0.0f;
        } else {
            const float pw = svk::fast_exp2(__builtin_fmaf(zp, a.c, -lp2));
            const float qw = svk::fast_exp2(__builtin_fmaf(zq, a.c, -lq2));
            const double d = st.resid_p ? (double)pw : (double)((float)st.wmul * pw - qw);
            const double r = d > 0.0 ? (qw > 0.0f ? d / (st.zr * (double)qw) : __builtin_inf()) : 0.0;
            ratio = r < 1.0 ? (float)r : 1.0f;
        }
        if (writer && a.diag.ratio) a.diag.ratio[(int64_t)b * t.N + (c - 1)] = ratio;
        if (st.u[c] < ratio) {   // accepted: continue at c
            st.path_x[st.depth] = st.x[c - 1];
            st.path_n[st.depth] = c;
            st.depth += 1;
            st.node = c;
            st.child = t.first_child[c];
            st.first = 1;
            st.resid_p = 1;
            continue;
        }
        // rejected: the residual becomes max(r - q, 0)
        st.wmul = st.resid_p ? 1.0 : st.wmul / (1.0 + st.zr);
        st.resid_p = 0;
        st.first = 0;
        st.mode = 0;
        const int nxt = t.next_sib[c];
        st.act = nxt >= 0 ? TREE_PASS : TREE_DRAW;
        st.child = nxt;
        return;
    }
    }
}

// Wavefront 0: decisions until a pass or the draw is needed.
template <int PES, int QES>
__device__ void tree_walk(const svh::VerifyArgs &a, const svh::TreeTopo &t, int b, TreeLDS &st, bool writer)
{
    if ((threadIdx.x & (svk::kWave - 1)) == 0) tree_decide(a, t, b, st, writer);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Wavefront 0: data checks, row statistics, uniforms; then the walk from the
// root.  A request with a data error gets its error outputs here.  Only the
// writer stores outputs and diagnostics (other workgroups of a request
// repeat the same steps for their own state).
template <int PES, int QES>
__device__ void tree_begin(const svh::VerifyArgs &a, const svh::TreeTopo &t, const float2 *__restrict__ part,
                           int nch1, int b, int32_t *__restrict__ nodes_out, uint32_t *__restrict__ errword,
                           TreeLDS &st, bool writer)
{
    const int lane = threadIdx.x & (svk::kWave - 1);
    const int N = t.N, NQ = t.NQ, D = t.D;
    const float nan = __builtin_nanf("");
    const int32_t x = lane < N ? a.draft[(int64_t)b * N + lane] : 0;
    const bool x_ok = x >= 0 && (int64_t)x < a.V;
    // node lane + 1's token logits under its parent's rows (decision-independent)
    if (lane < N && x_ok) {
        const int par = t.parent[lane + 1];
        st.zp[lane + 1] = svk::load_logit<PES>(a.p, tree_prow(t, b, par) * a.V + x);
        st.zq[lane + 1] = svk::load_logit<QES>(a.q, tree_qrow(t, b, par) * a.V + x);
    }
    bool bad = false;
    for (int n = lane; n <= N; n += svk::kWave) {
        bool bn = false;
        st.lp[n] = merge_row(part, tree_prow(t, b, n), nch1, bn);
        bad |= bn;
    }
    for (int j = lane; j < NQ; j += svk::kWave) {
        bool bq = false;
        st.lq[j] = merge_row(part, (int64_t)a.B * (N + 1) + (int64_t)b * NQ + j, nch1, bq);
        bad |= bq;
    }
    if (lane < N) {
        st.x[lane] = x;
        st.u[lane + 1] = a.uniforms ? a.uniforms[(int64_t)b * (N + 1) + lane]
                                    : svk::philox_uniform(a.seed, a.offset, (uint32_t)b, (uint32_t)(lane + 1), 0u);
    }
    uint32_t flags = 0;
    if (__ballot(lane < N && !x_ok)) flags = SV_FLAG_BAD_TOKEN;
    else if (__ballot(bad)) flags = SV_FLAG_BAD_ROW;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (writer) {
        for (int n = lane; n <= N; n += svk::kWave)
            if (a.diag.lse_p) a.diag.lse_p[(int64_t)b * (N + 1) + n] = flags ? nan : (float)(st.lp[n] * kLn2d);
        for (int j = lane; j < NQ; j += svk::kWave)
            if (a.diag.lse_q) a.diag.lse_q[(int64_t)b * NQ + j] = flags ? nan : (float)(st.lq[j] * kLn2d);
        for (int m = lane; m < N; m += svk::kWave)
            if (a.diag.ratio) a.diag.ratio[(int64_t)b * N + m] = nan;
    }
    if (flags) {
        if (writer) {
            for (int j = lane; j <= D; j += svk::kWave) a.out_tokens[(int64_t)b * (D + 1) + j] = -1;
            if (nodes_out)
                for (int j = lane; j < D; j += svk::kWave) nodes_out[(int64_t)b * D + j] = -1;
        }
        if (lane == 0) {
            if (writer) {
                a.accepted_len[b] = -1;
                if (a.diag.flags) a.diag.flags[b] = flags;
                atomicOr(errword, flags);
            }
            st.act = TREE_DONE;
        }
        return;
    }
    if (lane == 0) {
        st.node = 0;
        st.child = t.first_child[0];
        st.depth = 0;
        st.first = 1;
        st.resid_p = 1;
        st.flags = 0;
        st.zr = 1.0;
        st.wmul = 1.0;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    tree_walk<PES, QES>(a, t, b, st, writer);
}

// Wavefront 0, after the segment sums of the node's current weights are in
// sums[0, nseg): a pass gives the residual mass and the walk continues; the
// draw picks the token (or falls back to p once) and, if the writer, stores
// request b's outputs.
template <int PES, int QES>
__device__ void tree_consume(const svh::VerifyArgs &a, const svh::TreeTopo &t, int b, TreeLDS &st,
                             const float *sums, int nseg, int32_t *__restrict__ nodes_out,
                             uint32_t *__restrict__ errword, bool writer)
{
    const int lane = threadIdx.x & (svk::kWave - 1);
    const int node = st.node;
    const int mode = st.mode;
    if (st.act == TREE_PASS) {
        // mass of the residual weights: fixed-order fp64 sum of the segment sums
        const int per = (nseg + svk::kWave - 1) / svk::kWave;
        const int k0 = lane * per, k1 = k0 + per < nseg ? k0 + per : nseg;
        double loc = 0.0;
        for (int k = k0; k < k1; ++k) loc += (double)sums[k];
        const double Z = __shfl(svk::wave_inclusive_scan_d(loc), svk::kWave - 1, svk::kWave);
        if (lane == 0) {
            if (Z > 0.0) {
                st.zr = Z;
            } else {   // rounded to zero (positive in exact arithmetic): fall back to p
                st.flags |= SV_FLAG_RESID_ZERO;
                st.resid_p = 1;
                st.mode = 1;
                st.zr = 1.0;
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        tree_walk<PES, QES>(a, t, b, st, writer);
        return;
    }
    const char *prow = (const char *)a.p + tree_prow(t, b, node) * a.V * PES;
    const char *qrow = mode ? nullptr : (const char *)a.q + tree_qrow(t, b, node) * a.V * QES;
    const float lp2 = (float)st.lp[node];
    const float lq2 = mode ? 0.0f : (float)st.lq[t.qrow[node]];
    const float wm = (float)st.wmul;
    const float u2 = a.uniforms ? a.uniforms[(int64_t)b * (t.N + 1) + t.N]
                                : svk::philox_uniform(a.seed, a.offset, (uint32_t)b, 0u, 1u);
    double Z = 0.0;
    const int y = select_token_wave<PES, QES>(a, mode, wm, lp2, lq2, sums, nseg, prow, qrow, u2, Z);
    if (y < 0 && mode == 0) {
        // residual mass rounded to zero: draw from the node's p row
        if (lane == 0) {
            st.flags |= SV_FLAG_RESID_ZERO;
            st.mode = 1;
            st.wmul = 1.0;
        }
    } else {
        if (writer) {
            const uint32_t flags = st.flags | (y < 0 ? SV_FLAG_BAD_ROW : 0u);
            const int depth = st.depth, D = t.D;
            for (int j = lane; j <= D; j += svk::kWave)
                a.out_tokens[(int64_t)b * (D + 1) + j] =
                    y < 0 ? -1 : (j < depth ? st.path_x[j] : (j == depth ? y : -1));
            if (nodes_out)
                for (int j = lane; j < D; j += svk::kWave)
                    nodes_out[(int64_t)b * D + j] = (y >= 0 && j < depth) ? st.path_n[j] : -1;
            if (lane == 0) {
                a.accepted_len[b] = y < 0 ? -1 : depth;
                if (a.diag.flags) a.diag.flags[b] = flags;
                if (a.diag.resid_mass) a.diag.resid_mass[b] = (float)Z;
                if (flags) atomicOr(errword, flags);
            }
        }
        if (lane == 0) st.act = TREE_DONE;
    }
}

// The node's current weights: prow / qrow, mode, wmul and the row statistics.
struct TreeRows {
    const char *prow, *qrow;
    int mode;
    float wm, lp2, lq2;
};
template <int PES, int QES>
__device__ __forceinline__ TreeRows tree_rows(const svh::VerifyArgs &a, const svh::TreeTopo &t, int b,
                                              const TreeLDS &st)
{
    TreeRows r;
    const int node = st.node;
    r.mode = st.mode;
    r.prow = (const char *)a.p + tree_prow(t, b, node) * a.V * PES;
    r.qrow = r.mode ? nullptr : (const char *)a.q + tree_qrow(t, b, node) * a.V * QES;
    r.lp2 = (float)st.lp[node];
    r.lq2 = r.mode ? 0.0f : (float)st.lq[t.qrow[node]];
    r.wm = (float)st.wmul;
    return r;
}

// One workgroup per request walks its whole tree.
template <int PES, int QES, int NTT>
__global__ __launch_bounds__(NTT, 1) void k_tree(svh::VerifyArgs a, const svh::TreeTopo t,
                                              const float2 *__restrict__ part, int nch1, int nseg,
                                              int32_t *__restrict__ nodes_out, uint32_t *__restrict__ errword)
{
    __shared__ TreeLDS st;
    __shared__ float segsum[kTailMaxSeg];
    const int b = a.b0 + (int)blockIdx.x;
    const int wid = threadIdx.x / svk::kWave;
    if (wid == 0) tree_begin<PES, QES>(a, t, part, nch1, b, nodes_out, errword, st, true);
    __syncthreads();
    // every pass consumes one rejection or makes the draw (at most one retry
    // of the draw, from p): the loop ends well within this bound
    for (int it = 0; it < 2 * MAXG + 4; ++it) {
        if (st.act == TREE_DONE) return;
        const TreeRows r = tree_rows<PES, QES>(a, t, b, st);
        segment_sums<PES, QES, NTT / svk::kWave>(a, r.prow, r.qrow, r.mode, r.wm, r.lp2, r.lq2, nseg, segsum);
        __syncthreads();
        if (wid == 0) tree_consume<PES, QES>(a, t, b, st, segsum, nseg, nodes_out, errword, true);
        __syncthreads();
    }
}

// One round of the walk with S workgroups per request (blockIdx.x = S
// (b - b0) + s), for batches that leave most CUs idle with one workgroup per
// request.  Every workgroup of a request holds the same walk state: round 0
// starts the walk; a later round loads the state the previous round stored,
// reads the previous round's segment sums of all S workgroups and makes the
// same decisions.  Then, while a pass or the draw is pending, workgroup s
// sums its share of the segments.  State and segment sums are double
// buffered by round parity (a round reads one buffer and writes the other),
// workgroup 0 stores the state and writes every output.  The host launches
// enough rounds for the topology's longest sequence of passes.
template <int PES, int QES, int NTT>
__global__ __launch_bounds__(NTT, 1) void k_tree_round(svh::VerifyArgs a, const svh::TreeTopo t,
                                                    const float2 *__restrict__ part, int nch1, int nseg, int S,
                                                    int round, int max_batch, unsigned char *__restrict__ state_g,
                                                    float *__restrict__ seg_g, int32_t *__restrict__ nodes_out,
                                                    uint32_t *__restrict__ errword)
{
    __shared__ TreeLDS st;
    __shared__ float segsum[kTailMaxSeg];
    constexpr int W32 = (int)(sizeof(TreeLDS) / 4);
    static_assert(sizeof(TreeLDS) % 4 == 0 && sizeof(TreeLDS) <= svh::kTreeStateBytes, "tree state layout");
    const int s = (int)blockIdx.x % S;
    const int b = a.b0 + (int)blockIdx.x / S;
    const bool writer = s == 0;
    const int wid = threadIdx.x / svk::kWave;
    const int rd = (round + 1) & 1, wr = round & 1;   // buffers read and written by this round
    if (round == 0) {
        if (wid == 0) tree_begin<PES, QES>(a, t, part, nch1, b, nodes_out, errword, st, writer);
        __syncthreads();
    } else {
        const uint32_t *src = (const uint32_t *)(state_g + ((size_t)rd * max_batch + b) * svh::kTreeStateBytes);
        for (int i = threadIdx.x; i < W32; i += NTT) ((uint32_t *)&st)[i] = src[i];
        __syncthreads();
        if (st.act != TREE_DONE) {   // the same in every thread
            const float *sg = seg_g + ((size_t)rd * max_batch + b) * nseg;
            for (int k = threadIdx.x; k < nseg; k += NTT) segsum[k] = sg[k];
            __syncthreads();
            if (wid == 0) tree_consume<PES, QES>(a, t, b, st, segsum, nseg, nodes_out, errword, writer);
            __syncthreads();
        }
    }
    // stored every round, final states too, so the next round reads this one
    if (writer) {
        uint32_t *dst = (uint32_t *)(state_g + ((size_t)wr * max_batch + b) * svh::kTreeStateBytes);
        for (int i = threadIdx.x; i < W32; i += NTT) dst[i] = ((const uint32_t *)&st)[i];
    }
    if (st.act == TREE_DONE) return;
    // this round's pass (or draw): workgroup s sums segments [k0, k1)
    const int per = (nseg + S - 1) / S;
    const int k0 = s * per, k1 = k0 + per < nseg ? k0 + per : nseg;
    if (k0 >= k1) return;
    const TreeRows r = tree_rows<PES, QES>(a, t, b, st);
    segment_sums<PES, QES, NTT / svk::kWave>(a, r.prow, r.qrow, r.mode, r.wm, r.lp2, r.lq2, k1,
                                             seg_g + ((size_t)wr * max_batch + b) * nseg, k0);
}

template <int PES, int QES>
hipError_t tree_tail(sv_ctx *ctx, const svh::VerifyArgs &a, const svh::TreeTopo &t, int32_t *nodes_out,
                     hipStream_t s)
{
    // 512 threads: the walk, the segment sums and the draw together hold
    // about 200 VGPRs, which a 1024-thread workgroup (4 wavefronts per SIMD)
    // would spill
    const int slot = svh::prof_begin(ctx, s, SV_KERNEL_TAIL);
    // workgroups per request that one workgroup per CU allows, up to 8 (two
    // per CU measured no faster: the rounds' fixed costs dominate)
    int S = a.nb > 0 ? ctx->num_cu / a.nb : 1;
    S = S > 8 ? 8 : S;
    S = S > ctx->nseg ? ctx->nseg : S;
    if (S < 2) {
        hipLaunchKernelGGL((k_tree<PES, QES, NTT_NARROW>), dim3(a.nb), dim3(NTT_NARROW), 0, s, a, t,
                           (const float2 *)ctx->ws.part, ctx->nch1, ctx->nseg, nodes_out, ctx->ws.errword);
    } else {
        for (int round = 0; round < t.rounds; ++round)
            hipLaunchKernelGGL((k_tree_round<PES, QES, NTT_NARROW>), dim3(a.nb * S), dim3(NTT_NARROW), 0, s, a, t,
                               (const float2 *)ctx->ws.part, ctx->nch1, ctx->nseg, S, round, ctx->max_batch,
                               (unsigned char *)ctx->ws.tree_state, ctx->ws.tree_seg, nodes_out,
                               ctx->ws.errword);
    }
    svh::prof_end(ctx, s, slot);
    return hipGetLastError();
}

}  // namespace

namespace svh {

hipError_t launch_markov_verify_tail(sv_ctx *ctx, const VerifyArgs &a, const MarkovArgs &m, hipStream_t s)
{
    if (a.nb <= 0) return hipSuccess;
    return a.p_esize == 2 ? markov_verify_tail<2>(ctx, a, m, s) : markov_verify_tail<4>(ctx, a, m, s);
}

hipError_t launch_token_verify(sv_ctx *ctx, const VerifyArgs &a, hipStream_t s)
{
    if (a.nb <= 0) return hipSuccess;
    if (small_fits(ctx, a)) {
        if (a.p_esize == 2 && a.q_esize == 2) return token_single<2, 2>(ctx, a, s);
        if (a.p_esize == 2) return token_single<2, 4>(ctx, a, s);
        if (a.q_esize == 2) return token_single<4, 2>(ctx, a, s);
        return token_single<4, 4>(ctx, a, s);
    }
    const hipError_t e = launch_rowstats(ctx, a, s);
    if (e != hipSuccess) return e;
    return launch_token_tail(ctx, a, s);
}

hipError_t launch_token_tail(sv_ctx *ctx, const VerifyArgs &a, hipStream_t s)
{
    if (a.nb <= 0) return hipSuccess;
    if (a.p_esize == 2 && a.q_esize == 2) return token_tail<2, 2>(ctx, a, s);
    if (a.p_esize == 2) return token_tail<2, 4>(ctx, a, s);
    if (a.q_esize == 2) return token_tail<4, 2>(ctx, a, s);
    return token_tail<4, 4>(ctx, a, s);
}

hipError_t launch_block_tail(sv_ctx *ctx, const VerifyArgs &a, hipStream_t s)
{
    if (a.nb <= 0) return hipSuccess;
    if (a.p_esize == 2 && a.q_esize == 2) return block_tail<2, 2>(ctx, a, s);
    if (a.p_esize == 2) return block_tail<2, 4>(ctx, a, s);
    if (a.q_esize == 2) return block_tail<4, 2>(ctx, a, s);
    return block_tail<4, 4>(ctx, a, s);
}

hipError_t launch_tree_tail(sv_ctx *ctx, const VerifyArgs &a, const TreeTopo &t, int32_t *nodes_out, hipStream_t s)
{
    if (a.nb <= 0) return hipSuccess;
    if (ctx->nseg > kTailMaxSeg) return hipErrorInvalidValue;
    if (a.p_esize == 2 && a.q_esize == 2) return tree_tail<2, 2>(ctx, a, t, nodes_out, s);
    if (a.p_esize == 2) return tree_tail<2, 4>(ctx, a, t, nodes_out, s);
    if (a.q_esize == 2) return tree_tail<4, 2>(ctx, a, t, nodes_out, s);
    return tree_tail<4, 4>(ctx, a, t, nodes_out, s);
}

}  // namespace svh
