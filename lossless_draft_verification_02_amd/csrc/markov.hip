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
//   k_markov_gemm    z[b, n] = base[b, k, n] + sum_r U[x_{k-1}(b), r] Wt[n, r]
//                    computed transposed, z^T = Wt . U^T, with bf16 MFMA
//                    (16x16x32, fp32 accumulate).  Wt (the transition matrix
//                    stored vocabulary-major, V rows of R) gives the A operand
//                    straight from HBM: 16 bytes per lane per k-step, no LDS.
//                    The gathered U rows of up to 128 requests sit in LDS for
//                    the workgroup's lifetime and give the B operand.  Each
//                    accumulator lane holds 4 consecutive vocabulary entries
//                    of one request, so the epilogue adds the base logits and
//                    stores 16-byte runs of z without a detour through LDS,
//                    and reduces per (request, 128-token tile) the pair
//                    (max z*c, sum exp2(z*c - max)).  Workgroups of eight
//                    wavefronts (16 vocabulary rows each) loop over 128-token
//                    tiles; the next tile's Wt fragments and base logits are
//                    requested as soon as the current ones are consumed.
//   k_markov_select  one wavefront per request, no barriers: merge the tile
//                    pairs into the row's log-sum-exp, pick the tile holding
//                    u * Z by an fp64 wavefront scan, scan inside it for the
//                    token (inverse CDF in ascending token order).
#include "sv_device.h"
#include "sv_internal.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int NT = 512;                 // 8 wavefronts, 16 vocabulary rows each per tile
constexpr int NWAVE = NT / 64;
constexpr int TN = svh::kMarkovTileN;   // 128 vocabulary entries per tile
constexpr int MC = 128;                 // requests per workgroup (8 blocks of 16)
constexpr int MBLK = MC / 16;
constexpr int kGemmWGs = 512;           // two resident workgroups per compute unit

static_assert(TN == NWAVE * 16, "eight wavefronts of 16 vocabulary rows per tile");

__device__ __forceinline__ int prev_token(const svh::MarkovArgs &a, int k, int m)
{
    const int32_t x = k == 1 ? a.x0[m] : a.draft[(int64_t)m * a.gamma + (k - 2)];
    return (x < 0 || (int64_t)x >= a.V) ? 0 : x;   // invalid ids are flagged by the select
}

// The wavefront's A fragments of one tile: vocabulary row n = nrow0 + li,
// k-chunk 8 lg of each 32-wide k-step.  Rows past V read as zero.
template <int R>
__device__ __forceinline__ void load_wt(const svh::MarkovArgs &a, int64_t nrow0, int li, int lg,
                                        bf16x8 (&wa)[R / 32])
{
    const int64_t n = nrow0 + li;
    const uint16_t *row = a.W + (n < a.V ? n : 0) * R + 8 * lg;
#pragma unroll
    for (int s = 0; s < R / 32; ++s) wa[s] = n < a.V ? *(const bf16x8 *)(row + 32 * s) : bf16x8{};
}

// Base logits of the lane's outputs: requests m0 + 16 mb + li, vocabulary
// entries n .. n + 3 (bf16, packed in a uint2); -inf past V or past the batch.
__device__ __forceinline__ void load_base(const svh::MarkovArgs &a, int k, int m0, int mrows, int64_t n, int li,
                                          int vec, uint2 (&bv)[MBLK])
{
#pragma unroll
    for (int mb = 0; mb < MBLK; ++mb) {
        const int ml = 16 * mb + li;
        bv[mb] = make_uint2(0xFF80FF80u, 0xFF80FF80u);
        if (ml < mrows) {
            const uint16_t *brow = a.base + ((int64_t)(m0 + ml) * a.gamma + (k - 1)) * a.V;
            if (vec) {
                if (n < a.V) bv[mb] = *(const uint2 *)(brow + n);
            } else {
                uint16_t e[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) e[r] = n + r < a.V ? brow[n + r] : (uint16_t)0xFF80u;
                bv[mb] = make_uint2(e[0] | ((uint32_t)e[1] << 16), e[2] | ((uint32_t)e[3] << 16));
            }
        }
    }
}

template <int R>
__global__ __launch_bounds__(NT, 4) void k_markov_gemm(svh::MarkovArgs a, int k, float *__restrict__ zout,
                                                       int64_t zstride, float2 *__restrict__ tile_part,
                                                       int ntile, int vec)
{
    constexpr int KS = R / 32;
    constexpr int US = R + 8;              // LDS row stride (bf16): conflict-free 16-byte fragment reads
    constexpr int UCH = R / 8;             // 16-byte chunks per U row
    constexpr int UPT = MC * UCH / NT;     // chunks staged per thread
    static_assert(UPT >= 1 && MC * UCH % NT == 0, "U staging split");
    __shared__ __attribute__((aligned(16))) uint16_t Us[MC * US];
    __shared__ float2 red[NWAVE][MC];

    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int li = lane & 15, lg = lane >> 4;
    const int m0 = blockIdx.y * MC;
    const int mrows = a.B - m0 < MC ? a.B - m0 : MC;

    // first tile's Wt fragments and base logits, then the gathered U rows -> LDS
    int tile = blockIdx.x;
    bf16x8 wa[KS];
    uint2 bv[MBLK];
    load_wt<R>(a, (int64_t)tile * TN + 16 * wid, li, lg, wa);
    load_base(a, k, m0, mrows, (int64_t)tile * TN + 16 * wid + 4 * lg, li, vec, bv);
    {
        svk::u32x4 uv[UPT];
#pragma unroll
        for (int q = 0; q < UPT; ++q) {
            const int u = (int)threadIdx.x + q * NT;
            const int row = u / UCH, ch = u % UCH;
            uv[q] = svk::u32x4{0u, 0u, 0u, 0u};
            if (row < mrows) uv[q] = *(const svk::u32x4 *)(a.U + (int64_t)prev_token(a, k, m0 + row) * R + 8 * ch);
        }
#pragma unroll
        for (int q = 0; q < UPT; ++q) {
            const int u = (int)threadIdx.x + q * NT;
            *(svk::u32x4 *)(Us + (u / UCH) * US + 8 * (u % UCH)) = uv[q];
        }
    }
    svk::lds_barrier();

    for (; tile < ntile; tile += gridDim.x) {
        const int64_t n = (int64_t)tile * TN + 16 * wid + 4 * lg;   // the lane's first vocabulary entry
        // opaque to the optimiser, so the 16 row addresses below are rebuilt
        // per tile rather than held (and spilled) across the loop
        int li_t = li;
        asm volatile("" : "+v"(li_t));
        f32x4 acc[MBLK];
#pragma unroll
        for (int mb = 0; mb < MBLK; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
#pragma unroll
            for (int mb = 0; mb < MBLK; ++mb) {
                const bf16x8 bfr = *(const bf16x8 *)(Us + (16 * mb + li) * US + 32 * s + 8 * lg);
                acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[s], bfr, acc[mb], 0, 0, 0);
            }
        }
        // the fragments are consumed: fetch the next tile's into the same
        // registers, so the loads overlap the epilogue
        const int next = tile + (int)gridDim.x;
        if (next < ntile) load_wt<R>(a, (int64_t)next * TN + 16 * wid, li, lg, wa);

        // epilogue: lane holds z^T[n + r][16 mb + li]
#pragma unroll
        for (int mb = 0; mb < MBLK; ++mb) {
            const int ml = 16 * mb + li_t;
            const uint32_t b01 = bv[mb].x, b23 = bv[mb].y;
            float z[4];
            z[0] = acc[mb][0] + __uint_as_float(b01 << 16);
            z[1] = acc[mb][1] + __uint_as_float(b01 & 0xFFFF0000u);
            z[2] = acc[mb][2] + __uint_as_float(b23 << 16);
            z[3] = acc[mb][3] + __uint_as_float(b23 & 0xFFFF0000u);
            if (ml < mrows) {
                float *zrow = zout + (int64_t)(m0 + ml) * zstride;
                if (vec) {
                    if (n < a.V) *(float4 *)(zrow + n) = make_float4(z[0], z[1], z[2], z[3]);
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (n + r < a.V) zrow[n + r] = z[r];
                }
            }
            float zc[4];
            float mx = svk::neg_inf();
            bool bad = false;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                zc[r] = n + r < a.V ? z[r] * a.c : svk::neg_inf();
                mx = fmaxf(mx, zc[r]);
                bad |= zc[r] != zc[r];
            }
            // the four lanes li, li + 16, li + 32, li + 48 hold this request's 16 entries
            mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            float sm = 0.0f;
            if (mx != svk::neg_inf()) {
#pragma unroll
                for (int r = 0; r < 4; ++r) sm += svk::fast_exp2(zc[r] - mx);
            }
            if (bad) sm = __builtin_nanf("");   // a NaN entry poisons the row; the draw flags it
            sm += __shfl_xor(sm, 16, 64);
            sm += __shfl_xor(sm, 32, 64);
            if (lg == 0) red[wid][ml] = make_float2(mx, sm);
        }
        // the base logits are consumed: fetch the next tile's
        if (next < ntile) load_base(a, k, m0, mrows, (int64_t)next * TN + 16 * wid + 4 * lg, li_t, vec, bv);
        svk::lds_barrier();
        if ((int)threadIdx.x < mrows) {
            svk::MS t{red[0][threadIdx.x].x, red[0][threadIdx.x].y};
#pragma unroll
            for (int w = 1; w < NWAVE; ++w) t = svk::ms_merge(t, svk::MS{red[w][threadIdx.x].x, red[w][threadIdx.x].y});
            tile_part[(int64_t)(m0 + (int)threadIdx.x) * ntile + tile] = make_float2(t.m, t.s);
        }
        svk::lds_barrier();   // red[] is rewritten by the next tile
    }
}

constexpr int kSelWaves = 4;                                        // requests per workgroup
constexpr int kSelTilesPerLane = svh::kMarkovMaxTiles / 64;          // tile pairs held per lane

__device__ __forceinline__ int wave_min_i(int v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o, 64));
    return v;
}
__device__ __forceinline__ int wave_max_i(int v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
    return v;
}

__global__ __launch_bounds__(64 * kSelWaves) void k_markov_select(svh::MarkovArgs a, int k,
                                                                  const float *__restrict__ zin, int64_t zstride,
                                                                  const float2 *__restrict__ tile_part, int ntile,
                                                                  uint32_t *__restrict__ errword)
{
    const int lane = threadIdx.x & 63;
    const int b = blockIdx.x * kSelWaves + (int)(threadIdx.x >> 6);
    if (b >= a.B) return;   // whole wavefront; nothing below synchronises the workgroup
    const int64_t out = (int64_t)b * a.gamma + (k - 1);

    // independent loads first: the previous token and this lane's run of tile pairs
    const int32_t xprev = k == 1 ? a.x0[b] : a.draft[(int64_t)b * a.gamma + (k - 2)];
    const float2 *tp = tile_part + (int64_t)b * ntile;
    const int per = (ntile + 63) / 64;
    const int t0 = lane * per;
    float2 mine[kSelTilesPerLane];
#pragma unroll
    for (int q = 0; q < kSelTilesPerLane; ++q)
        mine[q] = (q < per && t0 + q < ntile) ? tp[t0 + q] : make_float2(svk::neg_inf(), 0.0f);
    const float u = a.uniforms ? a.uniforms[out]
                               : svk::philox_uniform(a.seed, a.offset, (uint32_t)b, (uint32_t)k, 2u);
    if (xprev < 0 || (int64_t)xprev >= a.V) {
        if (lane == 0) {
            a.draft[out] = -1;
            if (a.lse_q) a.lse_q[out] = __builtin_nanf("");
            atomicOr(errword, SV_FLAG_BAD_TOKEN);
        }
        return;
    }

    // row log-sum-exp2 from the tile pairs
    svk::MS acc{svk::neg_inf(), 0.0f};
#pragma unroll
    for (int q = 0; q < kSelTilesPerLane; ++q) acc = svk::ms_merge(acc, svk::MS{mine[q].x, mine[q].y});
    acc = svk::wave_merge(acc);
    const float lse2 = (acc.s > 0.0f && acc.m != svk::pos_inf() && acc.s == acc.s) ? acc.m + log2f(acc.s)
                                                                                    : __builtin_nanf("");
    if (lse2 != lse2) {
        if (lane == 0) {
            a.draft[out] = -1;
            if (a.lse_q) a.lse_q[out] = __builtin_nanf("");
            atomicOr(errword, SV_FLAG_BAD_ROW);
        }
        return;
    }

    // tile masses, fp64 prefix over the lanes' contiguous runs
    float wt[kSelTilesPerLane];
    double loc = 0.0;
#pragma unroll
    for (int q = 0; q < kSelTilesPerLane; ++q) {
        wt[q] = (q < per && t0 + q < ntile) ? mine[q].y * svk::fast_exp2(mine[q].x - lse2) : 0.0f;
        loc += (double)wt[q];
    }
    const double incl = svk::wave_inclusive_scan_d(loc);
    const double excl = incl - loc;
    const double Z = __shfl(incl, 63, 64);
    const float tf = __fmul_rn(u, (float)Z);
    int first = 0x7FFFFFFF, lastpos = -1;
    {
        double run = excl;
#pragma unroll
        for (int q = 0; q < kSelTilesPerLane; ++q) {
            if (q < per && t0 + q < ntile && wt[q] > 0.0f) {
                run += (double)wt[q];
                lastpos = t0 + q;
                if (first == 0x7FFFFFFF && (float)run > tf) first = t0 + q;
            }
        }
    }
    const int tstar = wave_min_i(first);
    const int tlast = wave_max_i(lastpos);
    const bool fallback = tstar == 0x7FFFFFFF;
    const int ts = fallback ? tlast : tstar;
    if (ts < 0) {   // no tile kept any mass
        if (lane == 0) {
            a.draft[out] = -1;
            if (a.lse_q) a.lse_q[out] = lse2 * svk::kLn2;
            atomicOr(errword, SV_FLAG_BAD_ROW);
        }
        return;
    }
    // cumulative mass before tile ts, from the lane that owns it
    double before_ts = excl;
#pragma unroll
    for (int q = 0; q < kSelTilesPerLane; ++q)
        if (q < per && t0 + q < ts) before_ts += (double)wt[q];
    const double tbase = __shfl(before_ts, ts / per, 64);

    // inside the tile: lane owns columns 2 lane, 2 lane + 1
    const int64_t c0 = (int64_t)ts * TN;
    const int ncols = (int)((a.V - c0) < TN ? (a.V - c0) : TN);
    const float *zr = zin + (int64_t)b * zstride + c0;
    const int j0 = 2 * lane, j1 = 2 * lane + 1;
    const float w0 = j0 < ncols ? svk::fast_exp2(zr[j0] * a.c - lse2) : 0.0f;
    const float w1 = j1 < ncols ? svk::fast_exp2(zr[j1] * a.c - lse2) : 0.0f;
    const double pair = (double)w0 + (double)w1;
    const double pincl = svk::wave_inclusive_scan_d(pair);
    const double pexcl = pincl - pair;
    int yb = 0x7FFFFFFF, yl = -1;
    if (w1 > 0.0f) {
        yl = j1;
        if (!fallback && (float)(tbase + pexcl + (double)w0 + (double)w1) > tf) yb = j1;
    }
    if (w0 > 0.0f) {
        if (yl < 0) yl = j0;
        if (!fallback && (float)(tbase + pexcl + (double)w0) > tf) yb = j0;
    }
    const int ybest = wave_min_i(yb);
    const int ylast = wave_max_i(yl);
    if (lane == 0) {
        const int j = ybest != 0x7FFFFFFF ? ybest : ylast;
        a.draft[out] = j >= 0 ? (int32_t)(c0 + j) : -1;
        if (a.lse_q) a.lse_q[out] = lse2 * svk::kLn2;
        if (j < 0) atomicOr(errword, SV_FLAG_BAD_ROW);
    }
}

template <int R>
hipError_t launch_positions(sv_ctx *ctx, const svh::MarkovArgs &a, hipStream_t s)
{
    const int ntile = ctx->ntile;
    const int gy = (a.B + MC - 1) / MC;
    int gx = kGemmWGs / gy;
    gx = gx < 1 ? 1 : (gx > ntile ? ntile : gx);
    // z rows of position k: the caller's q_logits [B, gamma, V], else a
    // workspace row per request
    const int64_t zstride = a.q_logits ? (int64_t)a.gamma * a.V : a.V;
    const int vec = (a.V % 4 == 0) && ((((uintptr_t)a.base) & 7) == 0) &&
                    ((((uintptr_t)(a.q_logits ? a.q_logits : ctx->ws.mk_q)) & 15) == 0);
    for (int k = 1; k <= a.gamma; ++k) {
        float *zk = a.q_logits ? a.q_logits + (int64_t)(k - 1) * a.V : ctx->ws.mk_q;
        int slot = svh::prof_begin(ctx, s, SV_KERNEL_MARKOV_GEMM);
        hipLaunchKernelGGL((k_markov_gemm<R>), dim3(gx, gy), dim3(NT), 0, s, a, k, zk, zstride, ctx->ws.mk_part,
                           ntile, vec);
        svh::prof_end(ctx, s, slot);
        slot = svh::prof_begin(ctx, s, SV_KERNEL_MARKOV_SELECT);
        hipLaunchKernelGGL(k_markov_select, dim3((a.B + kSelWaves - 1) / kSelWaves), dim3(64 * kSelWaves), 0, s,
                           a, k, (const float *)zk, zstride, (const float2 *)ctx->ws.mk_part, ntile,
                           ctx->ws.errword);
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
