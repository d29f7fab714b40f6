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
// One workgroup of 1024 threads: survival products in fp64 (sequential per
// request), an LDS bitonic sort of (S, candidate id) for up to 8192
// candidates, an fp64 block scan of the sorted survivals, and a parallel
// search for the first candidate that fails the test.
#include "sv_device.h"
#include "sv_internal.h"

namespace {

constexpr int NT = svh::kSchedThreads;
constexpr int NMAX = svh::kSchedMax;

__device__ __forceinline__ bool before(double ka, uint32_t ia, double kb, uint32_t ib)
{
    return ka > kb || (ka == kb && ia < ib);
}

__global__ __launch_bounds__(NT) void k_schedule(const float *__restrict__ conf, int B, int gamma,
                                                 double sps_k, int32_t *__restrict__ verify_len,
                                                 double *__restrict__ expected)
{
    __shared__ double key[NMAX];
    __shared__ uint16_t cid[NMAX];
    __shared__ int Lb[NMAX];
    __shared__ double scan[NT];
    __shared__ int kstop;

    const int n = B * gamma;
    int npow2 = 1;
    while (npow2 < n) npow2 <<= 1;

    for (int b = threadIdx.x; b < B; b += NT) {
        double S = 1.0;
        for (int i = 0; i < gamma; ++i) {
            float cf = conf[(int64_t)b * gamma + i];
            cf = cf > 0.0f ? (cf < 1.0f ? cf : 1.0f) : 0.0f;   // clamp, NaN -> 0
            S = S * (double)cf;
            key[b * gamma + i] = S;
            cid[b * gamma + i] = (uint16_t)(b * gamma + i);
        }
        Lb[b] = 0;
    }
    for (int k = n + threadIdx.x; k < npow2; k += NT) {
        key[k] = -1.0;
        cid[k] = 0xFFFF;
    }
    if (threadIdx.x == 0) kstop = n;
    __syncthreads();

    // bitonic sort into "before" order: S descending, then candidate id ascending
    for (int size = 2; size <= npow2; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int t = threadIdx.x; t < npow2 / 2; t += NT) {
                const int lo = 2 * stride * (t / stride) + (t % stride);
                const int hi = lo + stride;
                const bool up = (lo & size) == 0;
                const double klo = key[lo], khi = key[hi];
                const uint32_t ilo = cid[lo], ihi = cid[hi];
                const bool sw = up ? before(khi, ihi, klo, ilo) : before(klo, ilo, khi, ihi);
                if (sw) {
                    key[lo] = khi;
                    key[hi] = klo;
                    cid[lo] = (uint16_t)ihi;
                    cid[hi] = (uint16_t)ilo;
                }
            }
            __syncthreads();
        }
    }

    // fp64 prefix sums of sorted survivals: thread t owns [t*per, (t+1)*per)
    const int per = (n + NT - 1) / NT;
    const int k0 = threadIdx.x * per;
    const int k1 = k0 + per < n ? k0 + per : n;
    double loc = 0.0;
    for (int k = k0; k < k1; ++k) loc += key[k];
    double total;
    const double excl = svk::block_exclusive_scan_d<NT>(loc, scan, &total);
    {
        double E = (double)B + excl;
        for (int k = k0; k < k1; ++k) {
            const double rows = (double)B + (double)k;
            if (!(key[k] * (sps_k + rows) > E)) {
                atomicMin(&kstop, k);
                break;
            }
            E += key[k];
        }
    }
    __syncthreads();
    const int ks = kstop;
    for (int k = threadIdx.x; k < ks; k += NT) {
        const int id = cid[k];
        atomicMax(&Lb[id / gamma], id % gamma + 1);
    }
    if (expected) {
        // E of the admitted set: the prefix before the stopping candidate
        if (ks == n) {
            if (threadIdx.x == 0) *expected = (double)B + total;
        } else if (k0 <= ks && ks < k1) {
            double E = (double)B + excl;
            for (int k = k0; k < ks; ++k) E += key[k];
            *expected = E;
        }
    }
    __syncthreads();
    for (int b = threadIdx.x; b < B; b += NT) verify_len[b] = Lb[b];
}

}  // namespace

namespace svh {

hipError_t launch_schedule(sv_ctx *ctx, const float *conf, int B, int gamma, float sps_a,
                           float sps_k, int32_t *verify_len, double *expected, hipStream_t s)
{
    (void)sps_a;   // a positive scale of SPS does not move the maximum
    const int slot = prof_begin(ctx, s, SV_KERNEL_SCHEDULE);
    hipLaunchKernelGGL(k_schedule, dim3(1), dim3(NT), 0, s, conf, B, gamma, (double)sps_k,
                       verify_len, expected);
    const hipError_t e = hipGetLastError();
    prof_end(ctx, s, slot);
    return e;
}

}  // namespace svh
