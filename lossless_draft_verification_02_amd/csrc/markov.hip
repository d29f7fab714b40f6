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
//
// RNN head ("DeepSeek DSpark 详解", section 03, and "DSpark: DeepSeek's bet
// on speed that doesn't betray quality", section "A drafter that learns to
// doubt itself": the richer head variant carries a recurrent state over the
// block's prefix, so a draw can use more of it than the previous token).  Same contraction and draw, with the bf16 state hb_k as the left
// operand in place of U[x_{k-1}]: h_0 = 0, a_k = U[x_{k-1}] + A hb_{k-1}
// (A in linear-layer layout [out, in]; fp32, sequential fused multiply-adds
// over the state index starting from U[x_{k-1}]), hb_k = bf16(tanh(a_k)),
// round to nearest even.  hb_1 =
// bf16(tanh(U[x_0])) is formed wherever it is read; after drawing x_k the
// draw's workgroup computes hb_{k+1} for its request (a 256 x 256 product,
// A read from L2) and leaves it for the next position's contraction.
#include "sv_device.h"
#include "sv_internal.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int NT = 512;                 // 8 wavefronts
constexpr int NWAVE = NT / 64;
constexpr int TN = svh::kMarkovTileN;   // 128 vocabulary rows per tile (= the draw's tile)
constexpr int MC = 16 * NWAVE;          // 128 requests per workgroup: wavefront w owns 16 w .. 16 w + 15
constexpr int NVB = TN / 16;            // 16-row vocabulary blocks per tile

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ int prev_token(const svh::MarkovArgs &a, int k, int m)
{
    const int32_t x = k == 1 ? a.x0[m] : a.draft[(int64_t)m * a.gamma + (k - 2)];
    return (x < 0 || (int64_t)x >= a.V) ? 0 : x;   // invalid ids are flagged by the select
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Nearest bf16, ties to even; infinities pass, NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float x)
{
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u));
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint16_t rnn_first_state(const svh::MarkovArgs &a, int m, int j)
{
    int32_t x = a.x0[m];
    x = (x < 0 || (int64_t)x >= a.V) ? 0 : x;
    return f32_to_bf16(tanhf(bf16_to_f32(a.U[(int64_t)x * a.R + j])));
}

// The contraction's left operand for request m at position k, as the KS
// fragments of lane group lg (entries 8 lg + 32 s .. + 7): U[x_{k-1}] for the
// Markov head, the state hb_k for the RNN head.
template <int R>
__device__ __forceinline__ void head_fragments(const svh::MarkovArgs &a, int k, int m, int lg, bool act,
                                               bf16x8 (&ufr)[R / 32])
{
    constexpr int KS = R / 32;
    if (!act) {
#pragma unroll
        for (int s = 0; s < KS; ++s) ufr[s] = bf16x8{};
        return;
    }
    if (!a.A) {
        const uint16_t *urow = a.U + (int64_t)prev_token(a, k, m) * R + 8 * lg;
#pragma unroll
        for (int s = 0; s < KS; ++s) ufr[s] = *(const bf16x8 *)(urow + 32 * s);
    } else if (k == 1) {
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            uint16_t h[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) h[e] = rnn_first_state(a, m, 8 * lg + 32 * s + e);
            ufr[s] = __builtin_bit_cast(bf16x8, h);
        }
    } else {
        const uint16_t *hrow = a.hstate + (int64_t)m * R + 8 * lg;
#pragma unroll
        for (int s = 0; s < KS; ++s) ufr[s] = *(const bf16x8 *)(hrow + 32 * s);
    }
}

// RNN head, after request b's draw at position k (token xk, -1 if the draw
// failed), in two phases separated by the caller with a barrier over the
// NPART wavefronts that share the work (wavefront `part` takes state entries
// [part R / NPART, (part + 1) R / NPART)):
//   rnn_fill  hb_k (the state position k used) into the LDS scratch hs[R]
//             as floats, and to states_out;
//   rnn_next  for k < gamma, hb_{k+1} = bf16(tanh(U[xk] + A hb_k)) into
//             hstate: per entry j a sequential fp32 fma chain over r from
//             U[xk, j], A row j read as 16-byte runs (A in linear-layer
//             layout [out, in]), batches of loads issued ahead of the fmas.
// hstate[b] is read only in the first phase and written only in the second.
template <int R, int NPART>
__device__ void rnn_fill(const svh::MarkovArgs &a, int k, int b, float *hs, int part)
{
    constexpr int PER = R / NPART;
    const int lane = threadIdx.x & 63;
    const uint16_t *hrow = a.hstate + (int64_t)b * R;
#pragma unroll
    for (int q = 0; q < (PER + 63) / 64; ++q) {
        const int i = lane + 64 * q;
        if (i < PER) {
            const int j = part * PER + i;
            const uint16_t hbits = k == 1 ? rnn_first_state(a, b, j) : hrow[j];
            hs[j] = bf16_to_f32(hbits);
            if (a.states_out) a.states_out[((int64_t)b * a.gamma + (k - 1)) * R + j] = hbits;
        }
    }
}

template <int R, int NPART>
__device__ void rnn_next(const svh::MarkovArgs &a, int k, int b, int32_t xk, const float *hs, int part)
{
    constexpr int PER = R / NPART;
    constexpr int NC = R / 8;                     // 16-byte runs per A row
    constexpr int BATCH = NC < 16 ? NC : 16;
    if (k >= a.gamma) return;
    const int lane = threadIdx.x & 63;
    const int32_t x = (xk < 0 || (int64_t)xk >= a.V) ? 0 : xk;
#pragma unroll
    for (int q = 0; q < (PER + 63) / 64; ++q) {
        const int i = lane + 64 * q;
        if (i >= PER) break;
        const int j = part * PER + i;
        const uint16_t *arow = a.A + (int64_t)j * R;
        float acc = bf16_to_f32(a.U[(int64_t)x * R + j]);
        for (int c0 = 0; c0 < NC; c0 += BATCH) {
            uint4 w[BATCH];
#pragma unroll
            for (int c = 0; c < BATCH; ++c) w[c] = *(const uint4 *)(arow + 8 * (c0 + c));
#pragma unroll
            for (int c = 0; c < BATCH; ++c) {
                const uint32_t v[4] = {w[c].x, w[c].y, w[c].z, w[c].w};
                const float *h = hs + 8 * (c0 + c);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    acc = fmaf(h[2 * e], __uint_as_float(v[e] << 16), acc);
                    acc = fmaf(h[2 * e + 1], __uint_as_float(v[e] & 0xFFFF0000u), acc);
                }
            }
        }
        a.hstate[(int64_t)b * R + j] = f32_to_bf16(tanhf(acc));
    }
}

// One wavefront does both phases for its request (the non-fused draw).
template <int R>
__device__ void rnn_advance_wave(const svh::MarkovArgs &a, int k, int b, int32_t xk, float *hs)
{
    rnn_fill<R, 1>(a, k, b, hs, 0);
    // the wavefront's LDS writes are visible to its own later reads
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    rnn_next<R, 1>(a, k, b, xk, hs, 0);
}

// A tile of Wt (TN rows of R bf16) in LDS: row r's 16-byte chunk c sits at
// slot r * CH + (c ^ swz(r)), so the 16 rows of an A fragment read by one
// 16-lane group fall in different banks.
template <int R>
struct TileLayout {
    static constexpr int CH = R / 8;                        // 16-byte chunks per row
    static constexpr int SW = CH < 16 ? CH : 16;            // swizzle period
    static constexpr int BYTES = TN * R * 2;
    static constexpr int PER_WAVE = TN * CH / (NWAVE * 64); // copy instructions per wavefront
    static_assert(TN * CH % (NWAVE * 64) == 0, "whole copy instructions");
    __device__ static __forceinline__ int slot(int row, int c) { return row * CH + (c ^ (row & (SW - 1))); }
};

// Direct global -> LDS copy of Wt rows [n0, n0 + TN) into `dst`: each
// wavefront instruction fills 64 consecutive 16-byte slots (lane i -> slot
// base + i), fetching whichever global chunk the swizzle puts there.  Rows
// past V copy row V - 1; their outputs are never stored.
template <int R>
__device__ __forceinline__ void copy_tile(const svh::MarkovArgs &a, int64_t n0, unsigned char *dst, int wid, int lane)
{
    using TL = TileLayout<R>;
#pragma unroll
    for (int j = 0; j < TL::PER_WAVE; ++j) {
        const int base = (j * NWAVE + wid) * 64;
        const int S = base + lane;
        const int row = S / TL::CH, p = S % TL::CH;
        const int c = p ^ (row & (TL::SW - 1));
        int64_t n = n0 + row;
        n = n < a.V ? n : a.V - 1;
        __builtin_amdgcn_global_load_lds((const void *)(a.W + n * R + 8 * c), (lds_void *)(dst + base * 16), 16, 0, 0);
    }
}

// Base logits of the lane's outputs in one tile: request m, vocabulary
// entries n0 + 16 vb + 4 lg + r, as packed bf16 pairs; -inf past V or B.
__device__ __forceinline__ void load_base(const svh::MarkovArgs &a, int k, int m, int64_t n0, int lg, int vec,
                                          uint2 (&bv)[NVB])
{
    const uint16_t *brow = a.base + ((int64_t)(m < a.B ? m : 0) * a.gamma + (k - 1)) * a.V;
#pragma unroll
    for (int vb = 0; vb < NVB; ++vb) {
        const int64_t n = n0 + 16 * vb + 4 * lg;
        bv[vb] = make_uint2(0xFF80FF80u, 0xFF80FF80u);
        if (m < a.B) {
            if (vec) {
                if (n < a.V) bv[vb] = *(const uint2 *)(brow + n);
            } else {
                uint16_t e[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) e[r] = n + r < a.V ? brow[n + r] : (uint16_t)0xFF80u;
                bv[vb] = make_uint2(e[0] | ((uint32_t)e[1] << 16), e[2] | ((uint32_t)e[3] << 16));
            }
        }
    }
}

// Position k of every request (req == null), or position tau + 1 of each
// request whose scan ended in a rejection (req != null: the correction rows of
// the fused draft -> verification path; other requests are skipped).  zout
// may be null (no z rows stored) and tile_part may be null (no softmax pairs).
template <int R>
__global__ __launch_bounds__(NT, 2) void k_markov_gemm(svh::MarkovArgs a, int k, const svh::ReqG *__restrict__ req,
                                                       float *__restrict__ zout, int64_t zstride,
                                                       float2 *__restrict__ tile_part, int ntile, int vec)
{
    using TL = TileLayout<R>;
    constexpr int KS = R / 32;
    __shared__ __attribute__((aligned(16))) unsigned char wtile[2 * TL::BYTES];   // double-buffered tile ring

    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int li = lane & 15, lg = lane >> 4;
    const int m = blockIdx.y * MC + 16 * wid + li;   // the lane's request (B operand column)
    const bool wave_on = blockIdx.y * MC + 16 * wid < a.B;
    int km = k;                                        // the lane's position
    bool act = m < a.B;
    if (req && act) {
        const svh::ReqG r = req[m];
        act = r.flags == 0 && r.mode == 0;
        km = r.tau + 1;
    }

    // prologue: first tile's copy, the wavefront's U fragments, first base logits
    int tile = blockIdx.x;
    copy_tile<R>(a, (int64_t)tile * TN, wtile, wid, lane);
    bf16x8 ufr[KS];
    head_fragments<R>(a, km, m, lg, act, ufr);
    const int mb = act ? m : a.B;                      // load_base reads nothing for a.B
    uint2 bv[NVB];
    load_base(a, km, mb, (int64_t)tile * TN, lg, vec, bv);

    for (int it = 0; tile < ntile; ++it, tile += gridDim.x) {
        unsigned char *buf = wtile + (it & 1) * TL::BYTES;
        // this tile's copy (and base loads) landed for every wavefront, and
        // every wavefront finished reading the other buffer
        __builtin_amdgcn_s_waitcnt(0);
        svk::lds_barrier();
        const int next = tile + (int)gridDim.x;
        uint2 bn[NVB];
        if (next < ntile) {
            copy_tile<R>(a, (int64_t)next * TN, wtile + ((it + 1) & 1) * TL::BYTES, wid, lane);
            load_base(a, km, mb, (int64_t)next * TN, lg, vec, bn);
        }
        if (wave_on) {
            f32x4 acc[NVB];
#pragma unroll
            for (int vb = 0; vb < NVB; ++vb) acc[vb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KS; ++s) {
#pragma unroll
                for (int vb = 0; vb < NVB; ++vb) {
                    const int row = 16 * vb + li;
                    const bf16x8 afr = *(const bf16x8 *)(buf + 16 * TL::slot(row, 4 * s + lg));
                    acc[vb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr, ufr[s], acc[vb], 0, 0, 0);
                }
            }
            // epilogue: lane holds z^T[n0 + 16 vb + 4 lg + r][m]
            const int64_t n0 = (int64_t)tile * TN;
            float *zrow = zout ? zout + (int64_t)(act ? m : 0) * zstride : nullptr;
            float mx = svk::neg_inf();
            bool bad = false;
            float zc[NVB][4];
#pragma unroll
            for (int vb = 0; vb < NVB; ++vb) {
                const int64_t n = n0 + 16 * vb + 4 * lg;
                const uint32_t b01 = bv[vb].x, b23 = bv[vb].y;
                float z[4];
                z[0] = acc[vb][0] + __uint_as_float(b01 << 16);
                z[1] = acc[vb][1] + __uint_as_float(b01 & 0xFFFF0000u);
                z[2] = acc[vb][2] + __uint_as_float(b23 << 16);
                z[3] = acc[vb][3] + __uint_as_float(b23 & 0xFFFF0000u);
                if (zrow && act) {
                    if (vec) {
                        if (n < a.V) *(float4 *)(zrow + n) = make_float4(z[0], z[1], z[2], z[3]);
                    } else {
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            if (n + r < a.V) zrow[n + r] = z[r];
                    }
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    zc[vb][r] = n + r < a.V ? z[r] * a.c : svk::neg_inf();
                    mx = fmaxf(mx, zc[vb][r]);
                    bad |= zc[vb][r] != zc[vb][r];
                }
            }
            // lanes li, li + 16, li + 32, li + 48 hold request m's 128 entries
            mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            float sm = 0.0f;
            if (mx != svk::neg_inf()) {
#pragma unroll
                for (int vb = 0; vb < NVB; ++vb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) sm += svk::fast_exp2(zc[vb][r] - mx);
            }
            if (bad) sm = __builtin_nanf("");   // a NaN entry poisons the row; the draw flags it
            sm += __shfl_xor(sm, 16, 64);
            sm += __shfl_xor(sm, 32, 64);
            if (tile_part && lg == 0 && m < a.B) tile_part[(int64_t)m * ntile + tile] = make_float2(mx, sm);
        }
        if (next < ntile) {
#pragma unroll
            for (int vb = 0; vb < NVB; ++vb) bv[vb] = bn[vb];
        }
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

// State of one request's draw after the tile choice.
struct SelState {
    int32_t xprev;     // token sampled at the previous position (valid)
    float lse2;        // row log2-sum-exp2 of z * c
    float tf;          // fp32(u * fp32(Z)), Z the fp64 sum of the tile masses
    double tbase;      // cumulative mass before the chosen tile
    int ts;            // chosen tile
    int fallback;      // no cumulative mass exceeded tf: take the last positive token
};

// Tile choice for request b by one wavefront: merge the tile pairs into the
// row's log-sum-exp, fp64 prefix of the tile masses, the tile holding u * Z.
// Returns false when the request is finished (error outputs written).
__device__ bool select_tile(const svh::MarkovArgs &a, int k, const float2 *__restrict__ tile_part, int ntile,
                            uint32_t *__restrict__ errword, int b, SelState &st)
{
    const int lane = threadIdx.x & 63;
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
        return false;
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
        return false;
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
        return false;
    }
    // cumulative mass before tile ts, from the lane that owns it
    double before_ts = excl;
#pragma unroll
    for (int q = 0; q < kSelTilesPerLane; ++q)
        if (q < per && t0 + q < ts) before_ts += (double)wt[q];
    st.xprev = xprev;
    st.lse2 = lse2;
    st.tf = tf;
    st.tbase = __shfl(before_ts, ts / per, 64);
    st.ts = ts;
    st.fallback = fallback;
    return true;
}

// Token of the chosen tile (z values zr[0 .. 128)) by one wavefront: lane
// owns columns 2 lane, 2 lane + 1; fp64 prefix; outputs.  Returns the token
// (the same on every lane), -1 if none.
__device__ int32_t select_token_in_tile(const svh::MarkovArgs &a, int k, int b, const SelState &st,
                                     const float *zr, uint32_t *__restrict__ errword)
{
    const int lane = threadIdx.x & 63;
    const int64_t out = (int64_t)b * a.gamma + (k - 1);
    const int64_t c0 = (int64_t)st.ts * TN;
    const int ncols = (int)((a.V - c0) < TN ? (a.V - c0) : TN);
    const int j0 = 2 * lane, j1 = 2 * lane + 1;
    const float w0 = j0 < ncols ? svk::fast_exp2(zr[j0] * a.c - st.lse2) : 0.0f;
    const float w1 = j1 < ncols ? svk::fast_exp2(zr[j1] * a.c - st.lse2) : 0.0f;
    const double pair = (double)w0 + (double)w1;
    const double pincl = svk::wave_inclusive_scan_d(pair);
    const double pexcl = pincl - pair;
    int yb = 0x7FFFFFFF, yl = -1;
    if (w1 > 0.0f) {
        yl = j1;
        if (!st.fallback && (float)(st.tbase + pexcl + (double)w0 + (double)w1) > st.tf) yb = j1;
    }
    if (w0 > 0.0f) {
        if (yl < 0) yl = j0;
        if (!st.fallback && (float)(st.tbase + pexcl + (double)w0) > st.tf) yb = j0;
    }
    const int ybest = wave_min_i(yb);
    const int ylast = wave_max_i(yl);
    if (lane == 0) {
        const int j = ybest != 0x7FFFFFFF ? ybest : ylast;
        a.draft[out] = j >= 0 ? (int32_t)(c0 + j) : -1;
        if (a.lse_q) a.lse_q[out] = st.lse2 * svk::kLn2;
        if (a.lse2_out) a.lse2_out[out] = st.lse2;
        if (a.zx_out) a.zx_out[out] = j >= 0 ? zr[j] : __builtin_nanf("");
        if (j < 0) atomicOr(errword, SV_FLAG_BAD_ROW);
    }
    const int jj = ybest != 0x7FFFFFFF ? ybest : ylast;
    return jj >= 0 ? (int32_t)(c0 + jj) : -1;
}

// The draw with stored z rows: one wavefront per request, no barriers.
__global__ __launch_bounds__(64 * kSelWaves) void k_markov_select(svh::MarkovArgs a, int k,
                                                                  const float *__restrict__ zin, int64_t zstride,
                                                                  const float2 *__restrict__ tile_part, int ntile,
                                                                  uint32_t *__restrict__ errword)
{
    const int b = blockIdx.x * kSelWaves + (int)(threadIdx.x >> 6);
    if (b >= a.B) return;   // whole wavefront; nothing below synchronises the workgroup
    SelState st;
    if (!select_tile(a, k, tile_part, ntile, errword, b, st)) return;
    select_token_in_tile(a, k, b, st, zin + (int64_t)b * zstride + (int64_t)st.ts * TN, errword);
}

// The same draw for the RNN head, then the wavefront advances its request's
// state.
template <int R>
__global__ __launch_bounds__(64 * kSelWaves) void k_rnn_select(svh::MarkovArgs a, int k,
                                                               const float *__restrict__ zin, int64_t zstride,
                                                               const float2 *__restrict__ tile_part, int ntile,
                                                               uint32_t *__restrict__ errword)
{
    __shared__ float hs[kSelWaves][R];
    const int b = blockIdx.x * kSelWaves + (int)(threadIdx.x >> 6);
    if (b >= a.B) return;   // whole wavefront; nothing below synchronises the workgroup
    SelState st;
    if (!select_tile(a, k, tile_part, ntile, errword, b, st)) return;
    const int32_t xk = select_token_in_tile(a, k, b, st, zin + (int64_t)b * zstride + (int64_t)st.ts * TN, errword);
    rnn_advance_wave<R>(a, k, b, xk, hs[threadIdx.x >> 6]);
}

// The draw without stored z rows (fused path): one workgroup of 4 wavefronts
// per request.  Wavefront 0 chooses the tile; all four rebuild its 128 logits
// (two 16-row blocks each, every load issued before the MFMAs) with the
// contraction's own arithmetic -- same A rows, same k order, same base add --
// so they equal, bit for bit, the values reduced into the tile pairs;
// wavefront 0 then draws the token.
template <int R>
__global__ __launch_bounds__(256) void k_markov_select_fused(svh::MarkovArgs a, int k,
                                                            const float2 *__restrict__ tile_part, int ntile,
                                                            uint32_t *__restrict__ errword)
{
    constexpr int KS = R / 32;
    constexpr int VBW = NVB / 4;   // 16-row blocks per wavefront
    __shared__ SelState st;
    __shared__ int go;
    __shared__ float zt[TN];
    __shared__ float hs[R];   // RNN head: the request's state
    __shared__ int32_t xnew;   // the token drawn (RNN head)
    const int b = blockIdx.x;
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    if (wid == 0) {
        SelState s0;
        const bool ok = select_tile(a, k, tile_part, ntile, errword, b, s0);
        if (lane == 0) {
            go = ok;
            if (ok) st = s0;
        }
    }
    __syncthreads();
    if (!go) return;
    const int64_t c0 = (int64_t)st.ts * TN;
    const int ncols = (int)((a.V - c0) < TN ? (a.V - c0) : TN);
    const int li = lane & 15, lg = lane >> 4;
    bf16x8 ufr[KS], afr[VBW][KS];
    head_fragments<R>(a, k, b, lg, true, ufr);   // the request's operand row in every B column
#pragma unroll
    for (int v = 0; v < VBW; ++v) {
        const int64_t n = c0 + 16 * (VBW * wid + v) + li;
        const uint16_t *wrow = a.W + (n < a.V ? n : a.V - 1) * R + 8 * lg;
#pragma unroll
        for (int s = 0; s < KS; ++s) afr[v][s] = *(const bf16x8 *)(wrow + 32 * s);
    }
    const uint16_t *brow = a.base + ((int64_t)b * a.gamma + (k - 1)) * a.V + c0;
#pragma unroll
    for (int v = 0; v < VBW; ++v) {
        const int vb = VBW * wid + v;
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr[v][s], ufr[s], acc, 0, 0, 0);
        if (li == 0) {   // D[4 lg + r][0]: vocabulary row 16 vb + 4 lg + r of the tile
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int col = 16 * vb + 4 * lg + r;
                const uint32_t bits = col < ncols ? (uint32_t)brow[col] : 0xFF80u;
                zt[col] = acc[r] + __uint_as_float(bits << 16);
            }
        }
    }
    svk::lds_barrier();
    if (wid == 0) {
        const int32_t xk = select_token_in_tile(a, k, b, st, zt, errword);
        if (lane == 0) xnew = xk;
    }
    if (a.A) {   // RNN head: the four wavefronts advance the state together
        rnn_fill<R, 4>(a, k, b, hs, wid);
        __syncthreads();
        rnn_next<R, 4>(a, k, b, xnew, hs, wid);
    }
}

template <int R>
hipError_t launch_positions(sv_ctx *ctx, const svh::MarkovArgs &a, hipStream_t s)
{
    const int ntile = ctx->ntile;
    const int gy = (a.B + MC - 1) / MC;
    const size_t lds = 2 * (size_t)TileLayout<R>::BYTES;
    const int per_cu = lds <= 80 * 1024 ? 2 : 1;   // 160 KB of LDS per CU
    int gx = ctx->num_cu * per_cu / gy;
    gx = gx < 1 ? 1 : (gx > ntile ? ntile : gx);
    // z rows of position k: the caller's q_logits [B, gamma, V], else a
    // workspace row per request
    const int64_t zstride = a.q_logits ? (int64_t)a.gamma * a.V : a.V;
    const int vec = (a.V % 4 == 0) && ((((uintptr_t)a.base) & 7) == 0) &&
                    ((((uintptr_t)(a.q_logits ? a.q_logits : ctx->ws.mk_q)) & 15) == 0);
    for (int k = 1; k <= a.gamma; ++k) {
        float *zk = a.fused ? nullptr : (a.q_logits ? a.q_logits + (int64_t)(k - 1) * a.V : ctx->ws.mk_q);
        int slot = svh::prof_begin(ctx, s, SV_KERNEL_MARKOV_GEMM);
        hipLaunchKernelGGL((k_markov_gemm<R>), dim3(gx, gy), dim3(NT), 0, s, a, k, (const svh::ReqG *)nullptr, zk,
                           zstride, ctx->ws.mk_part, ntile, vec);
        svh::prof_end(ctx, s, slot);
        slot = svh::prof_begin(ctx, s, SV_KERNEL_MARKOV_SELECT);
        if (a.fused)
            hipLaunchKernelGGL((k_markov_select_fused<R>), dim3(a.B), dim3(256), 0, s, a, k,
                               (const float2 *)ctx->ws.mk_part, ntile, ctx->ws.errword);
        else if (a.A)
            hipLaunchKernelGGL((k_rnn_select<R>), dim3((a.B + kSelWaves - 1) / kSelWaves), dim3(64 * kSelWaves), 0,
                               s, a, k, (const float *)zk, zstride, (const float2 *)ctx->ws.mk_part, ntile,
                               ctx->ws.errword);
        else
            hipLaunchKernelGGL(k_markov_select, dim3((a.B + kSelWaves - 1) / kSelWaves), dim3(64 * kSelWaves), 0,
                               s, a, k, (const float *)zk, zstride, (const float2 *)ctx->ws.mk_part, ntile,
                               ctx->ws.errword);
        svh::prof_end(ctx, s, slot);
    }
    return hipGetLastError();
}

template <int R>
hipError_t launch_rebuild(sv_ctx *ctx, const svh::MarkovArgs &a, const svh::ReqG *req, float *qrec, hipStream_t s)
{
    const int ntile = ctx->ntile;
    const int gy = (a.B + MC - 1) / MC;
    const size_t lds = 2 * (size_t)TileLayout<R>::BYTES;
    const int per_cu = lds <= 80 * 1024 ? 2 : 1;
    int gx = ctx->num_cu * per_cu / gy;
    gx = gx < 1 ? 1 : (gx > ntile ? ntile : gx);
    const int vec = (a.V % 4 == 0) && ((((uintptr_t)a.base) & 7) == 0) && ((((uintptr_t)qrec) & 15) == 0);
    const int slot = svh::prof_begin(ctx, s, SV_KERNEL_MARKOV_REBUILD);
    hipLaunchKernelGGL((k_markov_gemm<R>), dim3(gx, gy), dim3(NT), 0, s, a, 0, req, qrec, a.V, (float2 *)nullptr,
                       ntile, vec);
    svh::prof_end(ctx, s, slot);
    return hipGetLastError();
}

}  // namespace

namespace svh {

hipError_t launch_markov_recompute(sv_ctx *ctx, const MarkovArgs &a, const ReqG *req, float *qrec, hipStream_t s)
{
    if (a.B <= 0 || a.gamma <= 0) return hipSuccess;
    switch (a.R) {
    case 32: return launch_rebuild<32>(ctx, a, req, qrec, s);
    case 64: return launch_rebuild<64>(ctx, a, req, qrec, s);
    case 128: return launch_rebuild<128>(ctx, a, req, qrec, s);
    case 256: return launch_rebuild<256>(ctx, a, req, qrec, s);
    default: return hipErrorInvalidValue;
    }
}

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
