// markov.hip -- Markov-head semi-autoregressive draft sampler.
//
// "DeepSeek Boosts Inference Speed by 85%" (kongchang.com), section "The
// First Ace", and "DeepSeek DSpark 详解" (zskr.cn), section 03: the parallel
// backbone gives base logits for every block position in one pass; a light
// sequential head then walks the block left to right, adding to position k's
// logits a rank-R (R = 256 on the pages) low-rank transition looked up from the
// token sampled at position k-1, and samples position k from the result.
//
// Per position k (strictly sequential; x_0 is the anchor token):
//   k_markov_gemm    grid (vocab tiles of 128, request blocks of 128):
//                    z[b, n] = base[b, k, n] + sum_r U[x_{k-1}(b), r] W[r, n]
//                    with bf16 MFMA (16x16x32, fp32 accumulate); the epilogue
//                    adds the base logits, writes z (fp32) and per (request,
//                    tile) the pair (max z*c, sum exp2(z*c - max)).
//   k_markov_select  one workgroup per request: merge the tile pairs into the
//                    row's log-sum-exp, pick the tile holding u * Z, scan it
//                    for the token (inverse CDF in ascending token order).
//
// Operand staging: the gathered U rows (A operand, 16 B per lane per k-step)
// are read straight from global memory into registers; the W tile is staged
// through LDS transposed to [n][k] so every B fragment is one 16-byte LDS read.
// The epilogue goes back through the same LDS space so base reads and z writes
// are row-contiguous.
#include "sv_device.h"
#include "sv_internal.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int NT = 256;                 // 4 wavefronts
constexpr int TN = svh::kMarkovTileN;   // 128 vocabulary columns per workgroup
constexpr int TM = 128;                 // requests per workgroup (32 per wavefront)
constexpr int RMAX = 256;
constexpr int WT_STRIDE_MAX = RMAX + 8;           // bf16 elements per transposed W row
constexpr int CT_STRIDE = TN + 4;                 // floats per epilogue row
constexpr int LDS_BYTES = (TN * WT_STRIDE_MAX * 2) > (TM * CT_STRIDE * 4)
                              ? (TN * WT_STRIDE_MAX * 2)
                              : (TM * CT_STRIDE * 4);

__device__ __forceinline__ int prev_token(const svh::MarkovArgs &a, int k, int m)
{
    const int32_t x = k == 1 ? a.x0[m] : a.draft[(int64_t)m * a.gamma + (k - 2)];
    return (x < 0 || (int64_t)x >= a.V) ? 0 : x;   // invalid ids are flagged by the select
}

template <int R>
__global__ __launch_bounds__(NT) void k_markov_gemm(svh::MarkovArgs a, int k, float *__restrict__ zout,
                                                    int64_t zstride, float2 *__restrict__ tile_part,
                                                    int ntile, int wvec)
{
    constexpr int KS = R / 32;            // MFMA k-steps
    constexpr int WTS = R + 8;            // transposed W row stride (bf16 elements)
    __shared__ __attribute__((aligned(16))) unsigned char lds[LDS_BYTES];
    __bf16 *Wt = (__bf16 *)lds;
    float *Ct = (float *)lds;

    const int tile = blockIdx.x;
    const int64_t n0 = (int64_t)tile * TN;
    const int ncols = (int)((a.V - n0) < TN ? (a.V - n0) : TN);
    const int m0 = blockIdx.y * TM;
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int li = lane & 15, lg = lane >> 4;

    // 1. W tile -> LDS, transposed: Wt[n][r] = W[r][n0 + n]
    if (wvec) {
        for (int u = threadIdx.x; u < (R / 4) * (TN / 8); u += NT) {
            const int kq = u / (TN / 8), n8 = u % (TN / 8);
            const int64_t col = n0 + 8 * n8;
            uint32_t w4[4][4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (col < a.V) {
                    const svk::u32x4 v = *(const svk::u32x4 *)(a.W + (int64_t)(4 * kq + j) * a.V + col);
                    w4[j][0] = v.x; w4[j][1] = v.y; w4[j][2] = v.z; w4[j][3] = v.w;
                } else {
                    w4[j][0] = w4[j][1] = w4[j][2] = w4[j][3] = 0u;
                }
            }
#pragma unroll
            for (int cc = 0; cc < 8; ++cc) {
                const int word = cc >> 1, hi = cc & 1;
                uint32_t e[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) e[j] = hi ? (w4[j][word] >> 16) : (w4[j][word] & 0xFFFFu);
                uint2 packed = make_uint2(e[0] | (e[1] << 16), e[2] | (e[3] << 16));
                *(uint2 *)(Wt + (8 * n8 + cc) * WTS + 4 * kq) = packed;
            }
        }
    } else {
        for (int u = threadIdx.x; u < R * TN; u += NT) {
            const int r = u / TN, n = u % TN;
            const int64_t col = n0 + n;
            const uint16_t bits = col < a.V ? a.W[(int64_t)r * a.V + col] : (uint16_t)0;
            ((uint16_t *)Wt)[n * WTS + r] = bits;
        }
    }

    // 2. A fragments: rows m0 + 32*wid + 16*mb + li, k = 32*ks + 8*lg .. +7
    bf16x8 afr[2][KS];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
        const int m = m0 + 32 * wid + 16 * mb + li;
        if (m < a.B) {
            const int x = prev_token(a, k, m);
            const uint16_t *urow = a.U + (int64_t)x * R;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) afr[mb][ks] = *(const bf16x8 *)(urow + 32 * ks + 8 * lg);
        } else {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) afr[mb][ks] = bf16x8{};
        }
    }
    __syncthreads();

    // 3. MFMA: each wavefront computes 32 rows x 128 columns
    f32x4 acc[2][TN / 16];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < TN / 16; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int nb = 0; nb < TN / 16; ++nb) {
            const bf16x8 bfr = *(const bf16x8 *)(Wt + (16 * nb + li) * WTS + 32 * ks + 8 * lg);
            acc[0][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr[0][ks], bfr, acc[0][nb], 0, 0, 0);
            acc[1][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr[1][ks], bfr, acc[1][nb], 0, 0, 0);
        }
    }
    __syncthreads();   // every wavefront is done with Wt

    // 4. accumulators -> LDS rows (lane holds D[4*lg + r][li] of each 16x16 block)
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < TN / 16; ++nb)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                Ct[(32 * wid + 16 * mb + 4 * lg + r) * CT_STRIDE + 16 * nb + li] = acc[mb][nb][r];
    __syncthreads();

    // 5. per row: z = base + acc, write z, tile (max, sum exp2)
    for (int rr = 0; rr < 32; ++rr) {
        const int mloc = 32 * wid + rr;
        const int m = m0 + mloc;
        if (m >= a.B) break;
        const uint16_t *brow = a.base + ((int64_t)m * a.gamma + (k - 1)) * a.V + n0;
        float *zrow = zout + (int64_t)m * zstride + n0;
        float zc[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int col = lane + 64 * h;
            zc[h] = svk::neg_inf();
            if (col < ncols) {
                const float z = Ct[mloc * CT_STRIDE + col] + __uint_as_float((uint32_t)brow[col] << 16);
                zrow[col] = z;
                zc[h] = z * a.c;
            }
        }
        float mx = fmaxf(zc[0], zc[1]);
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
        float s = 0.0f;
        if (mx != svk::neg_inf()) s = svk::fast_exp2(zc[0] - mx) + svk::fast_exp2(zc[1] - mx);
        // a NaN z poisons s (exp2(NaN) = NaN); keep it for the select to flag
        if (zc[0] != zc[0] || zc[1] != zc[1]) s = __builtin_nanf("");
        s = svk::wave_sum(s);
        if (lane == 0) tile_part[(int64_t)m * ntile + tile] = make_float2(mx, s);
    }
}

struct SelShared {
    double scan[NT];
    svk::MS red[NT / 64];
    float lse2;
    int tstar, tlast, ybest, ylast;
    double tbase;
};

__global__ __launch_bounds__(NT) void k_markov_select(svh::MarkovArgs a, int k, const float *__restrict__ zin,
                                                      int64_t zstride, const float2 *__restrict__ tile_part,
                                                      int ntile, uint32_t *__restrict__ errword)
{
    __shared__ SelShared sh;
    const int b = blockIdx.x;
    const int64_t out = (int64_t)b * a.gamma + (k - 1);
    const int32_t xprev = k == 1 ? a.x0[b] : a.draft[(int64_t)b * a.gamma + (k - 2)];
    if (xprev < 0 || (int64_t)xprev >= a.V) {
        if (threadIdx.x == 0) {
            a.draft[out] = -1;
            if (a.lse_q) a.lse_q[out] = __builtin_nanf("");
            atomicOr(errword, SV_FLAG_BAD_TOKEN);
        }
        return;
    }
    const float2 *tp = tile_part + (int64_t)b * ntile;
    // row log-sum-exp2 from the tile pairs
    svk::MS acc{svk::neg_inf(), 0.0f};
    for (int t = threadIdx.x; t < ntile; t += NT) acc = svk::ms_merge(acc, svk::MS{tp[t].x, tp[t].y});
    acc = svk::block_merge<NT>(acc, sh.red);
    if (threadIdx.x == 0) {
        sh.lse2 = (acc.s > 0.0f && acc.m != svk::pos_inf() && acc.s == acc.s) ? acc.m + log2f(acc.s)
                                                                                : __builtin_nanf("");
    }
    __syncthreads();
    const float lse2 = sh.lse2;
    if (lse2 != lse2) {
        if (threadIdx.x == 0) {
            a.draft[out] = -1;
            if (a.lse_q) a.lse_q[out] = __builtin_nanf("");
            atomicOr(errword, SV_FLAG_BAD_ROW);
        }
        return;
    }
    const float u = a.uniforms ? a.uniforms[out]
                               : svk::philox_uniform(a.seed, a.offset, (uint32_t)b, (uint32_t)k, 2u);

    // tile masses -> fp64 prefix, each thread owning a contiguous run of tiles
    const int per = (ntile + NT - 1) / NT;
    const int t0 = threadIdx.x * per;
    const int t1 = t0 + per < ntile ? t0 + per : ntile;
    double loc = 0.0;
    for (int t = t0; t < t1; ++t) loc += (double)(tp[t].y * svk::fast_exp2(tp[t].x - lse2));
    double Z;
    const double excl = svk::block_exclusive_scan_d<NT>(loc, sh.scan, &Z);
    const float tf = __fmul_rn(u, (float)Z);
    if (threadIdx.x == 0) {
        sh.tstar = 0x7FFFFFFF;
        sh.tlast = -1;
        sh.ybest = 0x7FFFFFFF;
        sh.ylast = -1;
    }
    __syncthreads();
    {
        double run = excl;
        for (int t = t0; t < t1; ++t) {
            const float wt = tp[t].y * svk::fast_exp2(tp[t].x - lse2);
            run += (double)wt;
            if (wt > 0.0f) {
                atomicMax(&sh.tlast, t);
                if ((float)run > tf) {
                    atomicMin(&sh.tstar, t);
                    break;
                }
            }
        }
    }
    __syncthreads();
    const bool fallback = sh.tstar == 0x7FFFFFFF;
    const int ts = fallback ? sh.tlast : sh.tstar;
    if (t0 <= ts && ts < t1) {
        double run = excl;
        for (int t = t0; t < ts; ++t) run += (double)(tp[t].y * svk::fast_exp2(tp[t].x - lse2));
        sh.tbase = run;
    }
    __syncthreads();
    // inside the tile: thread j < TN owns column j
    const int64_t c0 = (int64_t)ts * TN;
    const int ncols = (int)((a.V - c0) < TN ? (a.V - c0) : TN);
    float w = 0.0f;
    if ((int)threadIdx.x < ncols) w = svk::fast_exp2(zin[(int64_t)b * zstride + c0 + threadIdx.x] * a.c - lse2);
    double dummy;
    const double wexcl = svk::block_exclusive_scan_d<NT>((double)w, sh.scan, &dummy);
    if (w > 0.0f) {
        atomicMax(&sh.ylast, (int)threadIdx.x);
        if (!fallback && (float)(sh.tbase + wexcl + (double)w) > tf) atomicMin(&sh.ybest, (int)threadIdx.x);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        const int j = sh.ybest != 0x7FFFFFFF ? sh.ybest : sh.ylast;
        a.draft[out] = j >= 0 ? (int32_t)(c0 + j) : -1;
        if (a.lse_q) a.lse_q[out] = lse2 * svk::kLn2;
        if (j < 0) atomicOr(errword, SV_FLAG_BAD_ROW);
    }
}

template <int R>
hipError_t launch_positions(sv_ctx *ctx, const svh::MarkovArgs &a, hipStream_t s)
{
    const int ntile = ctx->ntile;
    const int wvec = (a.V % 8 == 0) && ((((uintptr_t)a.W) & 15) == 0);
    // z rows of position k: the caller's q_logits [B, gamma, V], else a
    // workspace row per request
    const int64_t zstride = a.q_logits ? (int64_t)a.gamma * a.V : a.V;
    for (int k = 1; k <= a.gamma; ++k) {
        float *zk = a.q_logits ? a.q_logits + (int64_t)(k - 1) * a.V : ctx->ws.mk_q;
        int slot = svh::prof_begin(ctx, s, SV_KERNEL_MARKOV_GEMM);
        hipLaunchKernelGGL((k_markov_gemm<R>), dim3(ntile, (a.B + TM - 1) / TM), dim3(NT), 0, s, a, k,
                           zk, zstride, ctx->ws.mk_part, ntile, wvec);
        svh::prof_end(ctx, s, slot);
        slot = svh::prof_begin(ctx, s, SV_KERNEL_MARKOV_SELECT);
        hipLaunchKernelGGL(k_markov_select, dim3(a.B), dim3(NT), 0, s, a, k, (const float *)zk, zstride,
                           (const float2 *)ctx->ws.mk_part, ntile, ctx->ws.errword);
        svh::prof_end(ctx, s, slot);
    }
    return hipGetLastError();
}

}  // namespace

namespace svh {

hipError_t launch_markov(sv_ctx *ctx, const MarkovArgs &a, hipStream_t s)
{
    if (a.B <= 0 || a.gamma <= 0) return hipSuccess;
    switch (a.R) {
    case 32: return launch_positions<32>(ctx, a, s);
    case 64: return launch_positions<64>(ctx, a, s);
    case 128: return launch_positions<128>(ctx, a, s);
    case 256: return launch_positions<256>(ctx, a, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace svh
