// sv_device.h -- device helpers shared by the gfx950 kernels of libspecverify.
//
// Arithmetic conventions of every kernel:
//  * logits are widened to fp32 and scaled once by c = log2(e) / T, so a row's
//    softmax is exp2(x*c - lse2) with lse2 = log2 sum_v exp2(x_v*c);
//  * partial row statistics are (m, s) pairs: m = max of x*c over the part,
//    s = sum exp2(x*c - m), merged with the usual rescaling;
//  * sums that decide an index are carried in fp64 across chunks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace svk {

constexpr int kWave = 64;
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }
__device__ __forceinline__ float pos_inf() { return __builtin_inff(); }
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11).  Only word 0 of the
// output block is used.  Ten rounds of: multiply counter words 0 and 2 by the
// Philox-4x32 multipliers, XOR the high halves with the other two words and the
// round key, permute; the key advances by the golden-ratio / sqrt(3)-1 Weyl
// increments between rounds.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t philox_word0(uint32_t c0, uint32_t c1, uint32_t c2,
                                                 uint32_t c3, uint32_t k0, uint32_t k1)
{
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint32_t a_lo = 0xD2511F53u * c0, a_hi = __umulhi(0xD2511F53u, c0);
        const uint32_t b_lo = 0xCD9E8D57u * c2, b_hi = __umulhi(0xCD9E8D57u, c2);
        const uint32_t n0 = b_hi ^ c1 ^ k0;
        const uint32_t n2 = a_hi ^ c3 ^ k1;
        c0 = n0;
        c1 = b_lo;
        c2 = n2;
        c3 = a_lo;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return c0;
}

// Uniform for (request, position, tag): 24 random bits scaled by 2^-24, so the
// value is exact in fp32 and lies in [0, 1 - 2^-24].
__device__ __forceinline__ float philox_uniform(uint64_t seed, uint64_t offset, uint32_t req,
                                                uint32_t pos, uint32_t tag)
{
    const uint32_t w = philox_word0(req, (pos & 0xFFFFu) | (tag << 16), (uint32_t)offset,
                                    (uint32_t)(offset >> 32), (uint32_t)seed,
                                    (uint32_t)(seed >> 32));
    return (float)(w >> 8) * 5.9604644775390625e-08f;
}

// ---------------------------------------------------------------------------
// Element access.  ESIZE 2 = bf16 (raw 16-bit), 4 = fp32.
// ---------------------------------------------------------------------------
template <int ESIZE>
__device__ __forceinline__ float load_logit(const void *base, int64_t idx)
{
    if constexpr (ESIZE == 2) {
        const uint32_t h = ((const uint16_t *)base)[idx];
        return __uint_as_float(h << 16);
    } else {
        return ((const float *)base)[idx];
    }
}

// 16-byte vector as a clang ext-vector (usable with the nontemporal builtins).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Widens one 16-byte vector into 16 / ESIZE floats.
template <int ESIZE>
__device__ __forceinline__ void widen(const u32x4 &v, float *out)
{
    if constexpr (ESIZE == 2) {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            out[2 * j] = __uint_as_float(w[j] << 16);
            out[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
        }
    } else {
        out[0] = __uint_as_float(v.x);
        out[1] = __uint_as_float(v.y);
        out[2] = __uint_as_float(v.z);
        out[3] = __uint_as_float(v.w);
    }
}

// A 16-byte vector whose every element is -inf (contributes nothing).
template <int ESIZE>
__device__ __forceinline__ u32x4 neg_inf_vec()
{
    const uint32_t w = ESIZE == 2 ? 0xFF80FF80u : 0xFF800000u;
    return u32x4{w, w, w, w};
}

// Workgroup barrier that orders LDS accesses only.  __syncthreads() is a
// workgroup-scope fence on every address space: it waits for all earlier
// global stores, and because loads and stores share one vector-memory counter
// that also drains every load issued before them (a prefetch included).  Use
// this where the workgroup communicates through LDS alone.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ---------------------------------------------------------------------------
// (max, sum-exp2) pairs.
// ---------------------------------------------------------------------------
struct MS {
    float m;   // max of x*c (scaled units), -inf if empty
    float s;   // sum exp2(x*c - m); NaN marks a NaN / +inf element
};

__device__ __forceinline__ MS ms_merge(MS a, MS b)
{
    const float M = fmaxf(a.m, b.m);
    if (M == neg_inf()) return {M, a.s + b.s};
    return {M, a.s * fast_exp2(a.m - M) + b.s * fast_exp2(b.m - M)};
}

__device__ __forceinline__ MS wave_merge(MS v)
{
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) {
        MS w;
        w.m = __shfl_xor(v.m, o, kWave);
        w.s = __shfl_xor(v.s, o, kWave);
        v = ms_merge(v, w);
    }
    return v;
}

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

__device__ __forceinline__ double wave_sum_d(double v)
{
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

// Block-wide merge for a 256-thread block; result valid in thread 0.
template <int NT>
__device__ __forceinline__ MS block_merge(MS v, MS *lds /* NT / 64 entries */)
{
    v = wave_merge(v);
    const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
    if (lane == 0) lds[wid] = v;
    __syncthreads();
    if (threadIdx.x == 0) {
        MS r = lds[0];
        for (int k = 1; k < NT / kWave; ++k) r = ms_merge(r, lds[k]);
        v = r;
    }
    return v;
}

template <int NT>
__device__ __forceinline__ float block_sum(float v, float *lds /* NT / 64 entries */)
{
    v = wave_sum(v);
    const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
    if (lane == 0) lds[wid] = v;
    __syncthreads();
    float r = 0.0f;
    if (threadIdx.x == 0)
        for (int k = 0; k < NT / kWave; ++k) r += lds[k];
    return r;
}

// Inclusive prefix of one double per lane across a wavefront (lane order).
__device__ __forceinline__ double wave_inclusive_scan_d(double v)
{
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const double t = __shfl_up(v, o, kWave);
        if (lane >= o) v += t;
    }
    return v;
}

// Exclusive prefix over the block of one double per thread (thread order):
// wavefront scans, then the wavefront totals in order.  Deterministic.
// Returns the exclusive prefix; *total gets the block total (all threads).
template <int NT>
__device__ __forceinline__ double block_exclusive_scan_d(double v, double *lds /* >= NT / 64 */,
                                                         double *total)
{
    const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
    const double incl = wave_inclusive_scan_d(v);
    double excl = __shfl_up(incl, 1, kWave);
    if (lane == 0) excl = 0.0;
    if (lane == kWave - 1) lds[wid] = incl;
    __syncthreads();
    double base = 0.0, tot = 0.0;
    for (int k = 0; k < NT / kWave; ++k) {
        const double t = lds[k];
        if (k < wid) base += t;
        tot += t;
    }
    __syncthreads();   // lds may be reused after return
    *total = tot;
    return base + excl;
}

}  // namespace svk
