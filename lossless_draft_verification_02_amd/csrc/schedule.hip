// schedule.hip -- hardware-aware prefix scheduler.
//
// "DeepSeek Boosts Inference Speed by 85%" (kongchang.com), section "The
// Third Ace", and "DeepSeek DSpark 详解" (zskr.cn), section 04: the survival
// probability of a draft prefix is the running product of the per-position
// conditional acceptance estimates; every round all extendable prefixes of all
// requests are ranked globally by survival and admitted one at a time while
// expected accepted tokens x engine step rate SPS(batch rows) keeps rising;
// admission stops at the first candidate that does not raise it, so it never
// looks past that point (the early stop the pages require for losslessness).
//
// Each request always verifies its correction / bonus row, so E starts at B
// and the verify batch at B rows.  With SPS(n) = a / (1 + n / K), admitting a
// candidate of survival s raises E * SPS iff s * (K + n) > E.
//
// With sequential temperature scaling the inputs are the confidence head's
// log-odds instead, and position i's estimate is the logistic of
// log-odds / T_i, each position with its own temperature ("DeepSeek Boosts
// Inference Speed by 85%", section "The Second Ace"; zskr.cn section 04);
// it is formed in fp64 where the survival products read it.
//
// Two kernels, handing over at the kernel boundary:
//   k_sched_rank   grid (candidate blocks) x (comparator blocks) of 256: the
//                  rank of candidate e in the order (S descending, id
//                  ascending) is the number of candidates that come before
//                  it; every workgroup counts one block of comparators for
//                  one block of candidates and adds its count atomically.
//                  Survival products are recomputed per block from the
//                  confidences, in the same sequential order everywhere.
//   k_sched_admit  one workgroup: scatter the candidates by rank into LDS
//                  (the sorted order), clear the ranks for the next call,
//                  fp64 block scan of the sorted survivals, find the first
//                  candidate that fails the test, set each request's length.
#include "sv_device.h"
#include "sv_internal.h"

namespace {

constexpr int RB = 256;                     // candidates (and comparators) per block
constexpr int NT = svh::kSchedThreads;      // admit workgroup
constexpr int NMAX = svh::kSchedMax;
constexpr int EPT = NMAX / NT;              // sorted slots per thread in the admit kernel
constexpr int CONF_MAX = RB + svh::kMaxGamma;

__device__ __forceinline__ double clamp01(double cf)
{
    return cf > 0.0 ? (cf < 1.0 ? cf : 1.0) : 0.0;   // NaN -> 0
}

// The confidence of candidate c (position c % gamma of its request): the
// input itself, or under temperature scaling the logistic of the input
// log-odds over that position's temperature; either is clamped to [0, 1].
__device__ __forceinline__ double candidate_confidence(const float *__restrict__ conf, int c, int gamma,
                                                       const svh::StsTemps &sts)
{
    const double v = (double)conf[c];
    if (!sts.on) return clamp01(v);
    const double odds = exp(-(v / (double)sts.t[c % gamma]));
    return clamp01(1.0 / (1.0 + odds));
}

// Survival products of candidates [e0, e0 + RB) into S[]: S(b, i) is the
// product of the confidences of positions 0..i of request b, formed left to
// right in fp64.  sconf is scratch of CONF_MAX doubles.
__device__ void block_survival(const float *__restrict__ conf, int n, int gamma, int e0,
                               const svh::StsTemps &sts, double *sconf, double *S)
{
    const int c0 = (e0 / gamma) * gamma;          // first position of the first request touched
    const int e1 = e0 + RB < n ? e0 + RB : n;
    for (int c = c0 + (int)threadIdx.x; c < e1; c += RB) sconf[c - c0] = candidate_confidence(conf, c, gamma, sts);
    __syncthreads();
    const int e = e0 + (int)threadIdx.x;
    if (e < n) {
        const int b0 = (e / gamma) * gamma;
        double s = 1.0;
        for (int c = b0; c <= e; ++c) s = s * sconf[c - c0];
        S[threadIdx.x] = s;
    }
    __syncthreads();
}

// How many of the comparators S[0..cn) come before (s, own index me):
// MODE 0, all earlier ids (S >= s); 1, all later ids (S > s); 2, the
// candidate's own block (S > s, or S == s at a smaller index).  Full blocks
// run unrolled so that many LDS reads are in flight.
template <int MODE>
__device__ __forceinline__ int count_before(const double *S, int cn, double s, int me)
{
    int cnt = 0;
    if (cn == RB) {
#pragma unroll 32
        for (int c = 0; c < RB; ++c)
            cnt += MODE == 0 ? S[c] >= s : MODE == 1 ? S[c] > s : (S[c] > s) || (S[c] == s && c < me);
    } else {
        for (int c = 0; c < cn; ++c)
            cnt += MODE == 0 ? S[c] >= s : MODE == 1 ? S[c] > s : (S[c] > s) || (S[c] == s && c < me);
    }
    return cnt;
}

__global__ __launch_bounds__(RB) void k_sched_rank(const float *__restrict__ conf, int n, int gamma,
                                                   const svh::StsTemps sts, int32_t *__restrict__ rank,
                                                   double *__restrict__ surv)
{
    __shared__ double Sx[RB], Sy[RB];
    __shared__ double sconf[CONF_MAX];
    const int bx = blockIdx.x, by = blockIdx.y;
    block_survival(conf, n, gamma, by * RB, sts, sconf, Sy);
    const int e = bx * RB + (int)threadIdx.x;
    double s;
    if (bx == by) {
        s = Sy[threadIdx.x];
    } else {
        block_survival(conf, n, gamma, bx * RB, sts, sconf, Sx);
        s = Sx[threadIdx.x];
    }
    if (e >= n) return;
    const int cn = n - by * RB < RB ? n - by * RB : RB;
    int cnt;
    if (by < bx) {          // every comparator id is smaller: ties come first
        cnt = count_before<0>(Sy, cn, s, 0);
    } else if (by > bx) {   // every comparator id is larger: ties come after
        cnt = count_before<1>(Sy, cn, s, 0);
    } else {
        cnt = count_before<2>(Sy, cn, s, (int)threadIdx.x);
        surv[e] = s;
    }
    if (cnt) atomicAdd(&rank[e], cnt);
}

__global__ __launch_bounds__(NT) void k_sched_admit(int n, int B, int gamma, double sps_k,
                                                    int32_t *__restrict__ rank, const double *__restrict__ surv,
                                                    int32_t *__restrict__ verify_len, double *__restrict__ expected,
                                                    uint32_t *__restrict__ errword)
{
    __shared__ double key[NMAX];
    __shared__ uint16_t cid[NMAX];
    __shared__ int Lb[NMAX];
    __shared__ double scan[NT / 64];
    __shared__ int kstop;

    const int t = threadIdx.x;
    for (int b = t; b < B; b += NT) Lb[b] = 0;
    if (t == 0) kstop = n;
    // scatter by rank: slot r of the sorted order; the ranks are a
    // permutation of [0, n), anything else is reported and dropped
    for (int e = t; e < n; e += NT) {
        const int r = rank[e];
        rank[e] = 0;
        if ((unsigned)r < (unsigned)n) {
            key[r] = surv[e];
            cid[r] = (uint16_t)e;
        } else {
            atomicOr(errword, SV_FLAG_BAD_ROW);
        }
    }
    __syncthreads();

    double k[EPT];
    int id[EPT];
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        const int e = EPT * t + j;
        k[j] = e < n ? key[e] : 0.0;
        id[j] = e < n ? (int)cid[e] : 0;
    }
    double loc = 0.0;
#pragma unroll
    for (int j = 0; j < EPT; ++j)
        if (EPT * t + j < n) loc += k[j];
    double total;
    const double excl = svk::block_exclusive_scan_d<NT>(loc, scan, &total);
    {
        double E = (double)B + excl;
#pragma unroll
        for (int j = 0; j < EPT; ++j) {
            const int kk = EPT * t + j;
            if (kk >= n) break;
            const double rows = (double)B + (double)kk;
            if (!(k[j] * (sps_k + rows) > E)) {
                atomicMin(&kstop, kk);
                break;
            }
            E += k[j];
        }
    }
    __syncthreads();
    const int ks = kstop;
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        const int kk = EPT * t + j;
        if (kk < ks) atomicMax(&Lb[id[j] / gamma], id[j] % gamma + 1);
    }
    if (expected) {
        // E of the admitted set: everything before the stopping candidate
        if (ks == n) {
            if (t == 0) *expected = (double)B + total;
        } else if (EPT * t <= ks && ks < EPT * t + EPT) {
            double E = (double)B + excl;
#pragma unroll
            for (int j = 0; j < EPT; ++j)
                if (EPT * t + j < ks) E += k[j];
            *expected = E;
        }
    }
    __syncthreads();
    for (int b = t; b < B; b += NT) verify_len[b] = Lb[b];
}

__global__ void k_sched_empty(int B, int32_t *__restrict__ verify_len, double *__restrict__ expected)
{
    for (int b = threadIdx.x; b < B; b += blockDim.x) verify_len[b] = 0;
    if (expected && threadIdx.x == 0) *expected = (double)B;
}

}  // namespace

namespace svh {

hipError_t launch_schedule(sv_ctx *ctx, const float *conf, const StsTemps &sts, int B, int gamma, float sps_a,
                           float sps_k, int32_t *verify_len, double *expected, hipStream_t s)
{
    (void)sps_a;   // a positive scale of SPS does not move the maximum
    const int n = B * gamma;
    const int slot = prof_begin(ctx, s, SV_KERNEL_SCHEDULE);
    if (n == 0) {
        hipLaunchKernelGGL(k_sched_empty, dim3(1), dim3(256), 0, s, B, verify_len, expected);
    } else {
        const int nb = (n + RB - 1) / RB;
        hipLaunchKernelGGL(k_sched_rank, dim3(nb, nb), dim3(RB), 0, s, conf, n, gamma, sts, ctx->ws.sched_rank,
                           ctx->ws.sched_surv);
        hipLaunchKernelGGL(k_sched_admit, dim3(1), dim3(NT), 0, s, n, B, gamma, (double)sps_k,
                           ctx->ws.sched_rank, (const double *)ctx->ws.sched_surv, verify_len, expected,
                           ctx->ws.errword);
    }
    const hipError_t e = hipGetLastError();
    prof_end(ctx, s, slot);
    return e;
}

}  // namespace svh
