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
//                    (16x16x32, fp32 accumulate).  One workgroup per CU of
//                    eight compute and four loader wavefronts walks 64-token
//                    tiles: the loaders copy each tile of Wt (the transition
//                    matrix stored vocabulary-major, V rows of R) and the
//                    tile's base logits straight from global memory into a
//                    three-slot LDS ring, two tiles ahead (the operand rows
//                    first: the previous draw, or before position 1 a copy
//                    kernel, left them contiguous); the compute
//                    wavefronts hold the U rows (or states) of the
//                    workgroup's 128 requests as B fragments in registers
//                    for the whole launch, read the A fragments from LDS
//                    (at rank 256 each feeds two MFMAs), add the base logits
//                    and reduce per (request, tile) the pair (max z*c,
//                    sum exp2(z*c - max)); z itself is stored only when the
//                    caller asks for the draft logits.
//   k_markov_draw    one 256-thread workgroup per request: the row maximum
//                    of the tile pairs, the tile masses relative to it and
//                    their fp64 prefix over the workgroup, the tile holding
//                    u * Z, then that tile's 64 logits (read back, or rebuilt
//                    by MFMA when no z rows are stored) scanned for the token
//                    (inverse CDF in ascending token order), and for the
//                    Markov head copies U[x_k] for the next position.  In the fused
//                    draft -> verification path the launch carries further
//                    workgroups that compute chunk statistics of the target
//                    rows (they do not depend on the draft), using the memory
//                    bandwidth the draw's few dependent round trips leave idle.
//
// RNN head ("DeepSeek DSpark 详解", section 03, and "DSpark: DeepSeek's bet
// on speed that doesn't betray quality", section "A drafter that learns to
// doubt itself": the richer head variant carries a recurrent state over the
// block's prefix, so a draw can use more of it than the previous token).
// Same contraction and draw, with the bf16 state hb_k as the left operand in
// place of U[x_{k-1}]: h_0 = 0, a_k = U[x_{k-1}] + A hb_{k-1} (A in
// linear-layer layout [out, in]; fp32, sequential fused multiply-adds over
// the state index starting from U[x_{k-1}]), hb_k = bf16(tanh(a_k)), round to
// nearest even.  hb_1 = bf16(tanh(U[x_0])) is written to the state buffer by
// a small kernel before position 1; after drawing x_k the draw's workgroup
// computes hb_{k+1} for its request (a 256 x 256 product, A read from L2)
// and leaves it for the next position's contraction.
#include <type_traits>

#include "sv_device.h"
#include "sv_internal.h"
#include "sv_rowstats.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int TN = svh::kMarkovTileN;   // vocabulary rows per tile (= the draw's tile)
constexpr int NVB = TN / 16;            // 16-row vocabulary blocks per tile
constexpr int NCW = 8;                  // contraction: compute wavefronts per workgroup
constexpr int NLW = 4;                  // contraction: loader wavefronts per workgroup
constexpr int NTG = (NCW + NLW) * 64;   // contraction workgroup
constexpr int MC = 128;                 // requests per contraction workgroup
constexpr int BASE_BYTES = MC * TN * 2; // base-logit tile: MC requests x TN tokens, bf16
static_assert(TN == 64, "one draw column per lane");

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

// hb_1 = bf16(tanh(U[x_0])) of every request into the state buffer, before
// position 1: the contraction and the draw then read every state from it,
// and neither carries the tanh code.
__global__ void k_rnn_first_state(svh::MarkovArgs a)
{
    const int b = blockIdx.x;
    for (int j = threadIdx.x; j < a.R; j += blockDim.x)
        a.hstate[(int64_t)b * a.R + j] = rnn_first_state(a, b, j);
}

// The contraction's left operand for request m at position k, as the KS
// fragments of lane group lg (entries 8 lg + 32 s .. + 7): U[x_{k-1}] for the
// Markov head, the state hb_k for the RNN head (hb_1 written beforehand).
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
            const uint16_t hbits = hrow[j];
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

// A tile of Wt (TN rows of R bf16) in LDS: row r's 16-byte chunk c sits at
// slot r * CH + (c ^ swz(r)), so the 16 rows of an A fragment read by one
// 16-lane group fall in different banks.
template <int R>
struct TileLayout {
    static constexpr int CH = R / 8;                        // 16-byte chunks per row
    static constexpr int SW = CH < 16 ? CH : 16;            // swizzle period
    static constexpr int BYTES = TN * R * 2;
    static constexpr int INSTR = TN * CH / 64;              // copy instructions (64 slots each)
    __device__ static __forceinline__ int slot(int row, int c) { return row * CH + (c ^ (row & (SW - 1))); }
};

// Copy instruction i of a Wt tile, rows [n0, n0 + TN) into `dst` (direct
// global -> LDS): lane l fills slot 64 i + l, fetching whichever global chunk
// the swizzle puts there.  Rows past V copy row V - 1; their outputs are
// never stored.
template <int R>
__device__ __forceinline__ void copy_w(const svh::MarkovArgs &a, int64_t n0, unsigned char *dst, int i, int lane)
{
    using TL = TileLayout<R>;
    const int S = 64 * i + lane;
    const int row = S / TL::CH, p = S % TL::CH;
    const int c = p ^ (row & (TL::SW - 1));
    int64_t n = n0 + row;
    n = n < a.V ? n : a.V - 1;
    __builtin_amdgcn_global_load_lds((const void *)(a.W + n * R + 8 * c), (lds_void *)(dst + 64 * i * 16), 16, 0, 0);
}

// The base-logit tile in LDS: request m's TN tokens are 8 chunks of 16 bytes,
// chunk c at slot 8 m + (c ^ (m & 7)).  Copy instruction i fills slots
// [64 i, 64 i + 64): requests 8 i .. 8 i + 7.  brow is lane's request row
// (the base row of its request and position); chunks past V fetch chunk 0.
__device__ __forceinline__ void copy_base(const uint16_t *brow, int64_t n0, int64_t V, unsigned char *dst, int i,
                                          int lane)
{
    const int S = 64 * i + lane;
    const int m = S >> 3, p = S & 7;
    int c = p ^ (m & 7);
    if (n0 + 8 * c >= V) c = 0;
    __builtin_amdgcn_global_load_lds((const void *)(brow + n0 + 8 * c), (lds_void *)(dst + 64 * i * 16), 16, 0, 0);
}

// The same tile from rows that are not 16-byte aligned: element loads,
// -inf past V, one 16-byte LDS store per lane.
__device__ __forceinline__ void copy_base_unaligned(const uint16_t *brow, int64_t n0, int64_t V, unsigned char *dst,
                                                    int i, int lane)
{
    const int S = 64 * i + lane;
    const int m = S >> 3, p = S & 7;
    const int c = p ^ (m & 7);
    uint16_t e[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int64_t n = n0 + 8 * c + q;
        e[q] = n < V ? brow[n] : (uint16_t)0xFF80u;
    }
    uint4 v;
    v.x = e[0] | ((uint32_t)e[1] << 16);
    v.y = e[2] | ((uint32_t)e[3] << 16);
    v.z = e[4] | ((uint32_t)e[5] << 16);
    v.w = e[6] | ((uint32_t)e[7] << 16);
    *(uint4 *)(dst + (size_t)S * 16) = v;
}

// Base logits n .. n + 3 (n = 16 vb + 4 lg, a multiple of 4) of request ml
// of the workgroup, from the LDS tile, as packed bf16 pairs.
__device__ __forceinline__ uint2 base_from_lds(const unsigned char *tile, int ml, int n)
{
    const int c = n >> 3, half = (n >> 2) & 1;
    return *(const uint2 *)(tile + (8 * ml + (c ^ (ml & 7))) * 16 + 8 * half);
}

// The loader wavefronts' side of the per-tile workgroup barrier.  Their
// copies write LDS behind the compiler's back: completion is their own
// explicit vmcnt wait before it, and the wavefront-scope fences only keep the
// compiler from moving a copy across the barrier (a workgroup-scope LDS
// fence here would make the compiler wait for every copy in flight, the next
// tile's included).
__device__ __forceinline__ void loader_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Waits until at most n of the calling wavefront's vector memory loads are
// outstanding (loads complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Max and sum over the four 16-lane rows (lanes l, l ^ 16, l ^ 32, l ^ 48):
// each swap hands a lane its own row's value and the partner row's, so the
// symmetric combination leaves the same result in every lane of the pair.
__device__ __forceinline__ float rows4_max(float v)
{
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
    const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}
__device__ __forceinline__ float rows4_sum(float v)
{
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(p[0]) + __uint_as_float(p[1]);
    const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

// How a contraction workgroup shares its work.  Compute wavefronts: each
// holds the B fragments of G request groups of 16 in registers for the whole
// launch and covers VBW of a tile's 16-row blocks, so every A fragment it
// reads from LDS feeds G MFMAs; the RP wavefronts of one request set split
// the tile's rows and combine their partial results through LDS.  Loader
// wavefronts only move data: each tile's Wt rows and base logits go straight
// from global memory into a three-slot LDS ring, two tiles ahead of the
// compute wavefronts, so no compute wavefront ever waits behind a memory
// instruction of its own.
template <int R>
struct GemmShape {
    static constexpr int G = R == 256 ? 2 : 1;      // request groups per compute wavefront
    static constexpr int NSET = MC / (16 * G);      // request sets
    static constexpr int RP = NCW / NSET;           // row parts of a tile
    static constexpr int VBW = NVB / RP;            // 16-row blocks per compute wavefront
    static constexpr int KS = R / 32;               // k-steps
    static constexpr int SLOT = TileLayout<R>::BYTES + BASE_BYTES;
    static constexpr int NSLOT = 3;
    static constexpr int W_PER = TileLayout<R>::INSTR / NLW;   // copy instructions per loader, per tile
    static constexpr int B_PER = BASE_BYTES / 1024 / NLW;
    static constexpr int PER = W_PER + B_PER;
    // the operand rows of the workgroup's MC requests, staged once in ring
    // slots 1-2 before tile 1 uses them: UCH 16-byte chunks per row, UI copy
    // instructions per loader
    static constexpr int UCH = R / 8;
    static constexpr int UI = MC * UCH / 64 / NLW;
    static_assert(NSET * RP == NCW && RP * VBW == NVB, "work split");
    static_assert(MC * R * 2 <= 2 * SLOT && (MC * UCH) % (64 * NLW) == 0, "operand rows fit two ring slots");
    static_assert(TileLayout<R>::INSTR % NLW == 0 && (BASE_BYTES / 1024) % NLW == 0, "whole copy instructions");
};

// Weight of one token in the correction / bonus draw of the fused
// verification ("Speculative Decoding: The Same Distribution, Twice as Fast",
// section 4: after a rejection the token comes from max(p - q, 0)
// normalised, after a full pass from p): with xp the target logit, z the
// draft logit and lp2, lq2 the rows' log2-sum-exp2 of x * c,
// w = max(wmul * 2^(xp c - lp2) - 2^(z c - lq2), 0), or 2^(xp c - lp2) for
// the bonus (mode 1).  The contraction's residual epilogue and the draw
// weigh a token through this one function, so their weights agree bit for
// bit.
__device__ __forceinline__ float resid_weight(float xp, float z, int mode, float wmul, float lp2, float lq2,
                                              float c)
{
    const float pw = svk::fast_exp2(__builtin_fmaf(xp, c, -lp2));
    if (mode) return pw;
    const float qw = svk::fast_exp2(__builtin_fmaf(z, c, -lq2));
    const float d = wmul * pw - qw;
    return d > 0.0f ? d : 0.0f;
}

// Four consecutive target logits n .. n + 3 of a p row (bf16 or fp32), as
// floats; -inf past V or for a null row.
template <int PES>
struct PQuad {
    typedef typename std::conditional<PES == 2, uint2, uint4>::type T;
};
template <int PES>
__device__ __forceinline__ typename PQuad<PES>::T p_quad(const char *prow, int n, int Vi, int vec)
{
    typename PQuad<PES>::T r;
    if constexpr (PES == 2) {
        r = make_uint2(0xFF80FF80u, 0xFF80FF80u);
        if (prow) {
            const uint16_t *row = (const uint16_t *)prow;
            if (vec) {
                if (n < Vi) r = *(const uint2 *)(row + n);
            } else {
                uint16_t e[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) e[q] = n + q < Vi ? row[n + q] : (uint16_t)0xFF80u;
                r = make_uint2(e[0] | ((uint32_t)e[1] << 16), e[2] | ((uint32_t)e[3] << 16));
            }
        }
    } else {
        const uint32_t ninf = 0xFF800000u;
        r = make_uint4(ninf, ninf, ninf, ninf);
        if (prow) {
            const uint32_t *row = (const uint32_t *)prow;
            if (vec) {
                if (n < Vi) r = *(const uint4 *)(row + n);
            } else {
                uint32_t e[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) e[q] = n + q < Vi ? row[n + q] : ninf;
                r = make_uint4(e[0], e[1], e[2], e[3]);
            }
        }
    }
    return r;
}
template <int PES>
__device__ __forceinline__ void p_quad_floats(const typename PQuad<PES>::T &v, float (&x)[4])
{
    if constexpr (PES == 2) {
        x[0] = __uint_as_float(v.x << 16);
        x[1] = __uint_as_float(v.x & 0xFFFF0000u);
        x[2] = __uint_as_float(v.y << 16);
        x[3] = __uint_as_float(v.y & 0xFFFF0000u);
    } else {
        x[0] = __uint_as_float(v.x);
        x[1] = __uint_as_float(v.y);
        x[2] = __uint_as_float(v.z);
        x[3] = __uint_as_float(v.w);
    }
}

// Residual mode of the contraction (the fused verification's correction /
// bonus rows): the target rows and the per-(request, tile) weight sums.
struct ResidArgs {
    const void *p;   // [B, gamma + 1, V] target logits
    float *tsum;     // [B, ntile] sums of resid_weight over each tile
};

// Draft mode (RES = 0): position k of every request; zout may be null (no z
// rows stored) and tile_part may be null (no softmax pairs).
// Residual mode (RES = the target logits' element size, 2 or 4): position
// tau + 1 of each request in req, the acceptance scan's results; every
// request it left without an error flag contributes its correction / bonus
// weights resid_weight over row tau + 1, summed per tile into ra.tsum; the
// contraction runs only for the requests that rejected (a bonus row needs p
// alone), and no z is stored.
//
// Per tile j of the workgroup (tiles blockIdx.x + j gridDim.x): the loader
// wavefronts request tile j + 2 into ring slot (j + 2) % 3 (the slot the
// compute wavefronts finished in iteration j - 1), then wait for tile
// j + 1's copies; the compute wavefronts multiply tile j out of slot j % 3
// (copied before the previous barrier), with the next k-step's A fragments
// read while the current k-step's MFMAs run, and reduce it.  One workgroup
// barrier per tile.  Per output the k-steps accumulate in ascending order
// (the draws rebuild their tiles the same way).
//
// STAGE (draft mode): the operand rows lie contiguous in hstate, one per
// request -- the RNN head's states hb_k, or the Markov head's U[x_{k-1}]
// that the previous position's draw (position 1: a small copy kernel) left
// there -- and the loaders copy each once into ring slots 1-2 ahead of tile
// 0; the compute wavefronts take them from there instead of each gathering
// its own.  The residual mode gathers U[x_tau] by token in the compute
// wavefronts.  (Gathering by token in the loaders instead put the token
// reads in front of their first tile.)
template <int R, int RES, bool STAGE>
__global__ __launch_bounds__(NTG, 1)
void k_markov_gemm(
    svh::MarkovArgs a, int k, const svh::ReqG *__restrict__ req, float *__restrict__ zout, int64_t zstride,
    float2 *__restrict__ tile_part, int ntile, int vec, int zvec, ResidArgs ra, int pvec)
{
    using TL = TileLayout<R>;
    using GS = GemmShape<R>;
    constexpr int G = GS::G, VBW = GS::VBW, KS = GS::KS, RP = GS::RP;
    __shared__ __attribute__((aligned(16))) unsigned char ring[GS::NSLOT * GS::SLOT];
    __shared__ svk::MS parts[RP > 1 ? 2 * RP * MC : 1];   // [tile parity][row part][request]: partials

    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const bool loader = wid >= NCW;
    const int Vi = (int)a.V;
    const int mbase = blockIdx.y * MC;   // first request of the workgroup
    int nt = 0;                          // tiles of the workgroup
    if ((int)blockIdx.x < ntile) nt = (ntile - 1 - (int)blockIdx.x) / (int)gridDim.x + 1;
    auto tile_of = [&](int j) { return (int)blockIdx.x + j * (int)gridDim.x; };
    auto slot_of = [&](int j) { return ring + (j % GS::NSLOT) * GS::SLOT; };

    if (loader) {
        // ---------------------------------------------------------------
        // loader wavefronts: Wt copy instructions lw, lw + NLW, ...; base
        // copy instructions likewise, each lane for one request row
        const int lw = wid - NCW;
        const uint16_t *brow[GS::B_PER];
#pragma unroll
        for (int q = 0; q < GS::B_PER; ++q) {
            const int i = lw + NLW * q;
            int m = mbase + ((64 * i + lane) >> 3);
            m = m < a.B ? m : a.B - 1;
            int km = k;
            if constexpr (RES != 0) {
                const svh::ReqG r = req[m];
                km = (r.flags == 0 && r.mode == 0) ? r.tau + 1 : 1;
            }
            brow[q] = a.base + ((int64_t)m * a.gamma + (km - 1)) * a.V;
        }
        auto issue = [&](int j) {
            const int64_t n0 = (int64_t)tile_of(j) * TN;
            unsigned char *sl = slot_of(j);
#pragma unroll
            for (int q = 0; q < GS::W_PER; ++q) copy_w<R>(a, n0, sl, lw + NLW * q, lane);
#pragma unroll
            for (int q = 0; q < GS::B_PER; ++q) {
                if (vec)
                    copy_base(brow[q], n0, a.V, sl + TL::BYTES, lw + NLW * q, lane);
                else
                    copy_base_unaligned(brow[q], n0, a.V, sl + TL::BYTES, lw + NLW * q, lane);
            }
        };
        if constexpr (STAGE) {
            // the operand rows first (each request's row of hstate once,
            // into ring slots 1-2, 16-byte chunks swizzled as the compute
            // wavefronts read them), then tile 0 alone: the compute
            // wavefronts take the rows into registers while tile 0 lands,
            // and tile 1 follows as soon as both are done
#pragma unroll
            for (int q = 0; q < GS::UI; ++q) {
                const int ml = (64 * (lw + NLW * q) + lane) / GS::UCH, pos = lane % GS::UCH;
                const int mm = mbase + ml < a.B ? mbase + ml : a.B - 1;
                const int c = pos ^ (ml & (GS::UCH - 1));
                __builtin_amdgcn_global_load_lds((const void *)(a.hstate + (int64_t)mm * R + 8 * c),
                                                 (lds_void *)(ring + GS::SLOT + 1024 * (lw + NLW * q)), 16, 0, 0);
            }
            if (nt > 0) issue(0);
            if (nt > 0 && vec) wait_vm<GS::PER>();   // the rows landed (tile 0 may be in flight)
            else __builtin_amdgcn_s_waitcnt(0);
            loader_barrier();                        // the compute wavefronts read the rows
            __builtin_amdgcn_s_waitcnt(0);           // tile 0 landed (element copies: their LDS stores too)
            loader_barrier();                        // rows read: slots 1-2 are free
            if (nt > 1) issue(1);
        } else {
            // tile 0 alone first: at the start every CU's first copies
            // compete for the memory system, and the compute wavefronts can
            // begin as soon as one tile has landed; tile 1 follows while they
            // multiply it
            if (nt > 0) issue(0);
            __builtin_amdgcn_s_waitcnt(0);   // tile 0 landed (element copies: their LDS stores too)
            if (nt > 1) issue(1);
            loader_barrier();
        }
        for (int j = 0; j < nt; ++j) {
            const bool more = j + 2 < nt;
            if (more) issue(j + 2);
            if (more && vec) wait_vm<GS::PER>();   // tile j + 1 landed
            else __builtin_amdgcn_s_waitcnt(0);
            loader_barrier();
        }
        return;
    }

    // -------------------------------------------------------------------
    // compute wavefronts
    const int li = lane & 15, lg = lane >> 4;
    const int set = wid % GS::NSET, rp = wid / GS::NSET;   // request set, row part
    const int vb0 = rp * VBW;                              // first 16-row block of the wavefront
    const int q0 = 16 * G * set;                           // first request of the set within the workgroup
    const bool wave_on = mbase + q0 < a.B;

    int m[G], km[G];
    bool act[G];
    // residual mode: the request's target row tau + 1 (null: no weights) and
    // its weight parameters
    [[maybe_unused]] const char *prow[G];
    [[maybe_unused]] float rmul[G], rlp2[G], rlq2[G];
    [[maybe_unused]] int rmode[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        m[g] = mbase + q0 + 16 * g + li;   // the lane's requests (B operand columns)
        km[g] = k;                         // and their positions
        act[g] = m[g] < a.B;
        if constexpr (RES != 0) {
            prow[g] = nullptr;
            rmode[g] = 1;
            rmul[g] = 1.0f;
            rlp2[g] = rlq2[g] = 0.0f;
            if (act[g]) {
                const svh::ReqG r = req[m[g]];
                act[g] = r.flags == 0 && r.mode == 0;
                km[g] = r.tau + 1;
                if (r.flags == 0) {
                    prow[g] = (const char *)ra.p + ((int64_t)m[g] * (a.gamma + 1) + r.tau) * a.V * RES;
                    rmode[g] = r.mode;
                    rmul[g] = r.wmul;
                    rlp2[g] = r.lp2;
                    rlq2[g] = r.lq2;
                }
            }
        }
    }
    bf16x8 ufr[G][KS];
    if constexpr (!STAGE) {
#pragma unroll
        for (int g = 0; g < G; ++g) head_fragments<R>(a, km[g], m[g], lg, act[g], ufr[g]);
    }

    // RP > 1: the pair (or weight sum) of (request, tile) from the row parts'
    // partials, written by the row-part-0 wavefronts once a barrier has passed
    auto merge_parts = [&](int par, int t) {
        if (RP > 1 && (RES != 0 || tile_part) && rp == 0 && lane < 16 * G) {
            const int mm = mbase + q0 + lane;
            if (mm < a.B) {
                if constexpr (RES != 0) {
                    float v = parts[(par * RP + 0) * MC + q0 + lane].s;
#pragma unroll
                    for (int r = 1; r < RP; ++r) v += parts[(par * RP + r) * MC + q0 + lane].s;
                    ra.tsum[(int64_t)mm * ntile + t] = v;
                } else {
                    svk::MS v = parts[(par * RP + 0) * MC + q0 + lane];
#pragma unroll
                    for (int r = 1; r < RP; ++r) v = svk::ms_merge(v, parts[(par * RP + r) * MC + q0 + lane]);
                    tile_part[(int64_t)mm * ntile + t] = make_float2(v.m, v.s);
                }
            }
        }
    };

    if constexpr (STAGE) {
        svk::lds_barrier();   // the operand rows landed in slots 1-2
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int ml = q0 + 16 * g + li;
#pragma unroll
            for (int s = 0; s < KS; ++s)
                ufr[g][s] = act[g] ? *(const bf16x8 *)(ring + GS::SLOT +
                                                       16 * (ml * GS::UCH + ((lg + 4 * s) ^ (ml & (GS::UCH - 1)))))
                                   : bf16x8{};
        }
    }
    svk::lds_barrier();   // tile 0 landed (STAGE: the rows are read, the loaders may refill slots 1-2)
    for (int j = 0; j < nt; ++j) {
        const int tile = tile_of(j);
        const unsigned char *sl = slot_of(j);
        const unsigned char *bt = sl + TL::BYTES;   // base-logit tile
        if (j > 0) merge_parts((j - 1) & 1, tile_of(j - 1));
        if (wave_on) {
            const int n0 = tile * TN;
            // residual mode: this tile's target logits, consumed by the epilogue
            typename PQuad<RES == 4 ? 4 : 2>::T pq[G][VBW];
            if constexpr (RES != 0) {
#pragma unroll
                for (int g = 0; g < G; ++g)
#pragma unroll
                    for (int v = 0; v < VBW; ++v)
                        pq[g][v] = p_quad<RES>(prow[g], n0 + 16 * (vb0 + v) + 4 * lg, Vi, pvec);
            }
            f32x4 acc[G][VBW];
#pragma unroll
            for (int g = 0; g < G; ++g)
#pragma unroll
                for (int v = 0; v < VBW; ++v) acc[g][v] = f32x4{0.f, 0.f, 0.f, 0.f};
            bf16x8 af[2][VBW];
#pragma unroll
            for (int v = 0; v < VBW; ++v) af[0][v] = *(const bf16x8 *)(sl + 16 * TL::slot(16 * (vb0 + v) + li, lg));
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const int cur = s & 1;
                if (s + 1 < KS) {
#pragma unroll
                    for (int v = 0; v < VBW; ++v)
                        af[cur ^ 1][v] = *(const bf16x8 *)(sl + 16 * TL::slot(16 * (vb0 + v) + li, 4 * (s + 1) + lg));
                }
#pragma unroll
                for (int g = 0; g < G; ++g)
#pragma unroll
                    for (int v = 0; v < VBW; ++v)
                        acc[g][v] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[cur][v], ufr[g][s], acc[g][v], 0, 0, 0);
            }
            // epilogue: lane holds z^T[n0 + 16 (vb0 + v) + 4 lg + r][m[g]]
            const bool full = n0 + TN <= Vi;
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const int ml = q0 + 16 * g + li;   // request within the workgroup
                float z[VBW][4];
#pragma unroll
                for (int v = 0; v < VBW; ++v) {
                    const uint2 bq = base_from_lds(bt, ml, 16 * (vb0 + v) + 4 * lg);
                    z[v][0] = acc[g][v][0] + __uint_as_float(bq.x << 16);
                    z[v][1] = acc[g][v][1] + __uint_as_float(bq.x & 0xFFFF0000u);
                    z[v][2] = acc[g][v][2] + __uint_as_float(bq.y << 16);
                    z[v][3] = acc[g][v][3] + __uint_as_float(bq.y & 0xFFFF0000u);
                }
                if constexpr (RES != 0) {
                    float sm = 0.0f;
#pragma unroll
                    for (int v = 0; v < VBW; ++v) {
                        const int n = n0 + 16 * (vb0 + v) + 4 * lg;
                        float xp[4];
                        p_quad_floats<RES == 4 ? 4 : 2>(pq[g][v], xp);
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            if (full || n + r < Vi)
                                sm += resid_weight(xp[r], z[v][r], rmode[g], rmul[g], rlp2[g], rlq2[g], a.c);
                    }
                    sm = rows4_sum(sm);
                    if (lg == 0) {
                        if (RP > 1)
                            parts[((j & 1) * RP + rp) * MC + ml] = svk::MS{0.0f, sm};
                        else if (m[g] < a.B)
                            ra.tsum[(int64_t)m[g] * ntile + tile] = sm;
                    }
                } else {
                    if (zout && act[g]) {
                        float *zrow = zout + (int64_t)m[g] * zstride;
#pragma unroll
                        for (int v = 0; v < VBW; ++v) {
                            const int n = n0 + 16 * (vb0 + v) + 4 * lg;
                            if (zvec && (full || n < Vi)) {
                                *(float4 *)(zrow + n) = make_float4(z[v][0], z[v][1], z[v][2], z[v][3]);
                            } else if (!zvec) {
#pragma unroll
                                for (int r = 0; r < 4; ++r)
                                    if (n + r < Vi) zrow[n + r] = z[v][r];
                            }
                        }
                    }
                    if (!tile_part) continue;
                    float mx = svk::neg_inf();
                    float zc[VBW][4];
#pragma unroll
                    for (int v = 0; v < VBW; ++v) {
                        const int n = n0 + 16 * (vb0 + v) + 4 * lg;
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            zc[v][r] = (full || n + r < Vi) ? z[v][r] * a.c : svk::neg_inf();
                            mx = fmaxf(mx, zc[v][r]);
                        }
                    }
                    mx = rows4_max(mx);   // over the request's 4 lanes: the wavefront's rows of the tile
                    // a NaN entry poisons the row (the draw flags it): through the
                    // exponentials when the maximum is finite, explicitly otherwise
                    float sm = 0.0f;
                    if (mx != svk::neg_inf()) {
#pragma unroll
                        for (int v = 0; v < VBW; ++v)
#pragma unroll
                            for (int r = 0; r < 4; ++r) sm += svk::fast_exp2(zc[v][r] - mx);
                    } else {
                        bool bad = false;
#pragma unroll
                        for (int v = 0; v < VBW; ++v)
#pragma unroll
                            for (int r = 0; r < 4; ++r) bad |= zc[v][r] != zc[v][r];
                        if (bad) sm = __builtin_nanf("");
                    }
                    sm = rows4_sum(sm);
                    if (lg == 0) {
                        if (RP > 1)
                            parts[((j & 1) * RP + rp) * MC + ml] = svk::MS{mx, sm};
                        else if (m[g] < a.B)
                            tile_part[(int64_t)m[g] * ntile + tile] = make_float2(mx, sm);
                    }
                }
            }
        }
        svk::lds_barrier();   // slot j % 3 is free again; tile j + 1 landed
    }
    if (nt > 0) merge_parts((nt - 1) & 1, tile_of(nt - 1));
}

#ifndef SV_MARKOV_RIDE_WGS_PER_CU
#define SV_MARKOV_RIDE_WGS_PER_CU 4   // riding target-row workgroups per CU in a draw launch
#endif
constexpr int kDrawThreads = 256;                                        // one workgroup per request
constexpr int kDrawWaves = kDrawThreads / 64;
constexpr int kDrawTilesPerThread = svh::kMarkovMaxTiles / kDrawThreads;  // tile pairs held per thread

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
__device__ __forceinline__ float wave_max_f(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

// State of one request's draw after the tile choice.
struct SelState {
    int32_t xprev;     // token sampled at the previous position (valid)
    float lse2;        // row log2-sum-exp2 of z * c
    float ref;         // row max of z * c: masses are exp2(z * c - ref)
    float tf;          // fp32(u * fp32(Z)), Z the fp64 sum of the tile masses
    double tbase;      // cumulative mass before the chosen tile
    int ts;            // chosen tile
    int fallback;      // no cumulative mass exceeded tf: take the last positive token
};

// Workgroup scratch of the tile choice.
struct DrawLDS {
    float wmax[kDrawWaves];
    int wbad[kDrawWaves];
    double scan[kDrawWaves];
    int wfirst[kDrawWaves], wlast[kDrawWaves];
    double wfirstb[kDrawWaves], wlastb[kDrawWaves];
};

// Tile choice for request b by the whole workgroup (every thread returns the
// same result): thread t holds tiles [t per, (t + 1) per); the row maximum
// M of the tile maxima; tile masses s exp2(m - M), their fp64 prefix in tile
// order (thread runs, then a deterministic block scan) and total Z; the row
// log2-sum-exp2 M + log2(Z); the first tile whose cumulative mass, rounded
// to binary32, exceeds fp32(u fp32(Z)) (else the last tile with mass).
// Returns false when the request is finished (error outputs written).
__device__ bool select_tile_wg(const svh::MarkovArgs &a, int k, const float2 *__restrict__ tile_part, int ntile,
                               uint32_t *__restrict__ errword, int b, DrawLDS &L, SelState &st)
{
    const int t = threadIdx.x, lane = t & 63, wid = t >> 6;
    const int64_t out = (int64_t)b * a.gamma + (k - 1);
    // independent loads first: the previous token and this thread's run of tile pairs
    const int32_t xprev = k == 1 ? a.x0[b] : a.draft[(int64_t)b * a.gamma + (k - 2)];
    const float2 *tp = tile_part + (int64_t)b * ntile;
    const int per = (ntile + kDrawThreads - 1) / kDrawThreads;
    const int t0 = t * per;
    float2 mine[kDrawTilesPerThread];
#pragma unroll
    for (int q = 0; q < kDrawTilesPerThread; ++q)
        mine[q] = (q < per && t0 + q < ntile) ? tp[t0 + q] : make_float2(svk::neg_inf(), 0.0f);
    const float u = a.uniforms ? a.uniforms[out]
                               : svk::philox_uniform(a.seed, a.offset, (uint32_t)b, (uint32_t)k, 2u);
    if (xprev < 0 || (int64_t)xprev >= a.V) {
        if (t == 0) {
            a.draft[out] = -1;
            if (a.lse_q) a.lse_q[out] = __builtin_nanf("");
            atomicOr(errword, SV_FLAG_BAD_TOKEN);
        }
        return false;
    }

    // row maximum; a NaN sum or a +inf maximum poisons the row
    float mloc = svk::neg_inf();
    bool bad = false;
#pragma unroll
    for (int q = 0; q < kDrawTilesPerThread; ++q) {
        mloc = fmaxf(mloc, mine[q].x);
        bad |= (mine[q].y != mine[q].y) || mine[q].x == svk::pos_inf();
    }
    mloc = wave_max_f(mloc);
    const bool wbad = __any(bad);
    if (lane == 0) {
        L.wmax[wid] = mloc;
        L.wbad[wid] = wbad;
    }
    __syncthreads();
    float M = L.wmax[0];
    bad = L.wbad[0];
#pragma unroll
    for (int w = 1; w < kDrawWaves; ++w) {
        M = fmaxf(M, L.wmax[w]);
        bad |= L.wbad[w] != 0;
    }

    // tile masses relative to M, fp64 prefix over the block
    float wt[kDrawTilesPerThread];
    double loc = 0.0;
#pragma unroll
    for (int q = 0; q < kDrawTilesPerThread; ++q) {
        wt[q] = mine[q].y > 0.0f ? mine[q].y * svk::fast_exp2(mine[q].x - M) : 0.0f;
        loc += (double)wt[q];
    }
    double Z;
    const double excl = svk::block_exclusive_scan_d<kDrawThreads>(loc, L.scan, &Z);
    const float lse2 = (!bad && M != svk::neg_inf() && Z > 0.0) ? M + log2f((float)Z) : __builtin_nanf("");
    if (lse2 != lse2) {
        if (t == 0) {
            a.draft[out] = -1;
            if (a.lse_q) a.lse_q[out] = __builtin_nanf("");
            atomicOr(errword, SV_FLAG_BAD_ROW);
        }
        return false;
    }

    // the first tile past the threshold, and the last tile with mass, each
    // with the cumulative mass before it
    const float tf = __fmul_rn(u, (float)Z);
    int first = 0x7FFFFFFF, last = -1;
    double firstb = 0.0, lastb = 0.0;
    {
        double run = excl;
#pragma unroll
        for (int q = 0; q < kDrawTilesPerThread; ++q) {
            if (wt[q] > 0.0f) {
                const double before = run;
                run += (double)wt[q];
                last = t0 + q;
                lastb = before;
                if (first == 0x7FFFFFFF && (float)run > tf) {
                    first = t0 + q;
                    firstb = before;
                }
            }
        }
    }
    // runs are contiguous in thread order: the lowest thread with a first
    // tile holds the workgroup's first, the highest with mass its last
    {
        const uint64_t hasf = __ballot(first != 0x7FFFFFFF), hasl = __ballot(last >= 0);
        const int lf = hasf ? __builtin_ctzll(hasf) : 0;
        const int ll = hasl ? 63 - __builtin_clzll(hasl) : 0;
        const int fw = __shfl(first, lf, 64), lw = __shfl(last, ll, 64);
        const double fbw = __shfl(firstb, lf, 64), lbw = __shfl(lastb, ll, 64);
        if (lane == 0) {
            L.wfirst[wid] = hasf ? fw : 0x7FFFFFFF;
            L.wfirstb[wid] = fbw;
            L.wlast[wid] = hasl ? lw : -1;
            L.wlastb[wid] = lbw;
        }
    }
    __syncthreads();
    int ts = 0x7FFFFFFF, tl = -1;
    double tb = 0.0, tlb = 0.0;
#pragma unroll
    for (int w = 0; w < kDrawWaves; ++w) {
        if (ts == 0x7FFFFFFF && L.wfirst[w] != 0x7FFFFFFF) {
            ts = L.wfirst[w];
            tb = L.wfirstb[w];
        }
        if (L.wlast[w] >= 0) {
            tl = L.wlast[w];
            tlb = L.wlastb[w];
        }
    }
    const bool fallback = ts == 0x7FFFFFFF;
    if (tl < 0) {   // no tile kept any mass
        if (t == 0) {
            a.draft[out] = -1;
            if (a.lse_q) a.lse_q[out] = lse2 * svk::kLn2;
            atomicOr(errword, SV_FLAG_BAD_ROW);
        }
        return false;
    }
    st.xprev = xprev;
    st.lse2 = lse2;
    st.ref = M;
    st.tf = tf;
    st.tbase = fallback ? tlb : tb;
    st.ts = fallback ? tl : ts;
    st.fallback = fallback;
    return true;
}

// Token of the chosen tile (z values zr[0 .. TN)) by one wavefront: lane
// owns column lane; masses exp2(z c - ref) as the tile choice's; fp64
// prefix; outputs.  Returns the token (the same on every lane), -1 if none.
__device__ int32_t select_token_in_tile(const svh::MarkovArgs &a, int k, int b, const SelState &st,
                                        const float *zr, uint32_t *__restrict__ errword)
{
    const int lane = threadIdx.x & 63;
    const int64_t out = (int64_t)b * a.gamma + (k - 1);
    const int64_t c0 = (int64_t)st.ts * TN;
    const int ncols = (int)((a.V - c0) < TN ? (a.V - c0) : TN);
    const int j0 = lane;
    const float w0 = j0 < ncols ? svk::fast_exp2(zr[j0] * a.c - st.ref) : 0.0f;
    const double pincl = svk::wave_inclusive_scan_d((double)w0);
    const double pexcl = pincl - (double)w0;
    int yb = 0x7FFFFFFF, yl = -1;
    if (w0 > 0.0f) {
        yl = j0;
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

// The riding workgroups of one draw launch: workgroup w of nw takes items
// first + w, first + w + nw, ... below end; item i is chunk i % nch1 of
// target row i / nch1, reduced exactly as the row-statistics pass reduces it
// (the same per-thread loads and fold order, the same workgroup merge) into
// part[i].  When a chunk is one load batch per thread (bf16 chunks of at
// most 32 KB) the next item's batch is requested before the current one is
// folded, so each workgroup keeps its loads in flight through the
// arithmetic.
__device__ void ride_items(const svh::RowRide &r, int64_t V, int64_t first, int64_t end, int64_t nw)
{
    static_assert(kDrawThreads == svh::kRowstatsThreads, "the row-statistics workgroup shape");
    constexpr int NB = svh::kRowstatsNB, NT = kDrawThreads;
    __shared__ svk::MS red[2][NT / 64];   // alternating: a wavefront may start the next merge early
    const bool nt = SV_ROWSTATS_NT_LOADS;
    const int tid = threadIdx.x;
    int par = 0;
    auto plan = [&](int64_t item, auto esize) {
        constexpr int ES = decltype(esize)::value;
        const int64_t row = item / r.nch1;
        const int64_t e0 = (item - row * r.nch1) * r.chunk1;
        const int64_t e1 = e0 + r.chunk1 < V ? e0 + r.chunk1 : V;
        return svk::chunk_plan<ES>((const char *)r.p + row * V * ES, e0, e1);
    };
    auto emit = [&](int64_t item, svk::MS t) {
        const svk::MS tot = svk::block_merge<NT>(t, red[par]);
        par ^= 1;
        if (tid == 0) r.part[item] = make_float2(tot.m, tot.s);
    };
    if (r.pes == 2 && r.chunk1 * 2 + 16 <= (int64_t)NT * NB * 16) {
        using E2 = std::integral_constant<int, 2>;
        if (first >= end) return;
        svk::ChunkPlan<2> cur = plan(first, E2{});
        svk::u32x4 raw[NB];
        svk::load_batch<2, NB, NT>(cur, tid, nt, raw);
        for (int64_t item = first; item < end; item += nw) {
            const int64_t nx = item + nw;
            svk::ChunkPlan<2> nxt = cur;
            svk::u32x4 rawn[NB];
            if (nx < end) {
                nxt = plan(nx, E2{});
                svk::load_batch<2, NB, NT>(nxt, tid, nt, rawn);
            }
            svk::RunStats st = svk::run_start();
            svk::fold_batch<2, NB>(raw, r.c, st);
            emit(item, svk::run_finish<2>(cur, r.c, tid, st));
            cur = nxt;
#pragma unroll
            for (int j = 0; j < NB; ++j) raw[j] = rawn[j];
        }
    } else {
        for (int64_t item = first; item < end; item += nw) {
            svk::MS t;
            if (r.pes == 2) {
                const svk::ChunkPlan<2> pl = plan(item, std::integral_constant<int, 2>{});
                t = svk::thread_stats<2, NB, NT>(pl.rowptr, pl.e0, pl.e1, r.c, nt, tid);
            } else {
                const svk::ChunkPlan<4> pl = plan(item, std::integral_constant<int, 4>{});
                t = svk::thread_stats<4, NB, NT>(pl.rowptr, pl.e0, pl.e1, r.c, nt, tid);
            }
            emit(item, t);
        }
    }
}

// Markov head: the next position's operand row U[x_k] (row 0 for an invalid
// or missing token, as prev_token reads it), copied by wavefront 0 to the
// request's row of hstate, where the next contraction's loaders take it.
template <int R>
__device__ __forceinline__ void stage_next_row(const svh::MarkovArgs &a, int b, int32_t xk)
{
    static_assert(R % 8 == 0 && R / 8 <= 64, "one 16-byte chunk per lane");
    const int lane = threadIdx.x & 63;
    const int64_t x = (xk < 0 || (int64_t)xk >= a.V) ? 0 : xk;
    if (lane < R / 8)
        ((uint4 *)(a.hstate + (int64_t)b * R))[lane] = ((const uint4 *)(a.U + x * R))[lane];
}

// Markov head, before position 1: U[x_0] of every request into hstate, so
// that position 1's contraction stages its operand rows as the later ones
// do.  One wavefront per request.
template <int R>
__global__ __launch_bounds__(64) void k_markov_first_rows(svh::MarkovArgs a)
{
    stage_next_row<R>(a, (int)blockIdx.x, a.x0[blockIdx.x]);
}

// The draw at position k: one workgroup of four wavefronts per request.  All
// threads choose the tile; its 64 logits come from the stored z rows (zin)
// or, without them (fused path), are rebuilt by the four wavefronts (two
// 16-row blocks each) with the contraction's own arithmetic -- same A rows,
// same k order, same base add -- so they equal, bit for bit, the values
// reduced into the tile pairs; the B fragments of that rebuild are requested
// before the tile choice.  Wavefront 0 then draws the token; for the RNN head
// the four wavefronts advance the request's state.
template <int R, bool RIDE>
__global__ __launch_bounds__(kDrawThreads) void k_markov_draw(svh::MarkovArgs a, int k,
                                                              const float *__restrict__ zin, int64_t zstride,
                                                              const float2 *__restrict__ tile_part, int ntile,
                                                              uint32_t *__restrict__ errword, int64_t ride0,
                                                              int64_t ride_n)
{
    constexpr int KS = R / 32;
    constexpr int VBW = NVB / kDrawWaves;   // 16-row blocks per wavefront
    if (RIDE && (int)blockIdx.x >= a.B) {   // workgroups past the draws: riding target-row chunks
        ride_items(a.ride, a.V, ride0 + ((int64_t)blockIdx.x - a.B), ride0 + ride_n, (int64_t)gridDim.x - a.B);
        return;
    }
    __shared__ DrawLDS L;
    __shared__ float zt[TN];
    __shared__ float hs[R];    // RNN head: the request's state
    __shared__ int32_t xnew;   // the token drawn (RNN head)
    const int b = blockIdx.x;
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int li = lane & 15, lg = lane >> 4;
    bf16x8 ufr[KS];
    if (!zin) head_fragments<R>(a, k, b, lg, true, ufr);   // the request's operand row in every B column
    SelState st;
    // Markov head with a state buffer: the draw leaves the next position's
    // operand row there
    const bool stage = !a.A && a.hstate && k < a.gamma;
    if (!select_tile_wg(a, k, tile_part, ntile, errword, b, L, st)) {   // the same in every thread
        if (stage && wid == 0) stage_next_row<R>(a, b, -1);
        return;
    }
    const int64_t c0 = (int64_t)st.ts * TN;
    const int ncols = (int)((a.V - c0) < TN ? (a.V - c0) : TN);
    if (zin) {
        if ((int)threadIdx.x < ncols) zt[threadIdx.x] = zin[(int64_t)b * zstride + c0 + threadIdx.x];
    } else {
        bf16x8 afr[VBW][KS];
#pragma unroll
        for (int v = 0; v < VBW; ++v) {
            const int64_t n = c0 + 16 * (VBW * wid + v) + li;
            const uint16_t *wrow = a.W + (n < a.V ? n : a.V - 1) * R + 8 * lg;
#pragma unroll
            for (int s = 0; s < KS; ++s) afr[v][s] = *(const bf16x8 *)(wrow + 32 * s);
        }
        // base logits of the lane's outputs, requested with the A rows (an
        // in-row address for every column; -inf replaces those past V)
        const uint16_t *brow = a.base + ((int64_t)b * a.gamma + (k - 1)) * a.V + c0;
        uint32_t bbits[VBW][4];
#pragma unroll
        for (int v = 0; v < VBW; ++v)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int col = 16 * (VBW * wid + v) + 4 * lg + r;
                bbits[v][r] = brow[col < ncols ? col : 0];
            }
#pragma unroll
        for (int v = 0; v < VBW; ++v) {
            const int vb = VBW * wid + v;
            f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KS; ++s)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr[v][s], ufr[s], acc, 0, 0, 0);
            if (li == 0) {   // D[4 lg + r][0]: vocabulary row 16 vb + 4 lg + r of the tile
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int col = 16 * vb + 4 * lg + r;
                    const uint32_t bits = col < ncols ? bbits[v][r] : 0xFF80u;
                    zt[col] = acc[r] + __uint_as_float(bits << 16);
                }
            }
        }
    }
    svk::lds_barrier();
    if (wid == 0) {
        const int32_t xk = select_token_in_tile(a, k, b, st, zt, errword);
        if (lane == 0) xnew = xk;
        if (stage) stage_next_row<R>(a, b, xk);
    }
    if (a.A) {   // RNN head: the four wavefronts advance the state together
        rnn_fill<R, kDrawWaves>(a, k, b, hs, wid);
        __syncthreads();
        rnn_next<R, kDrawWaves>(a, k, b, xnew, hs, wid);
    }
}

// ---------------------------------------------------------------------------
// Correction / bonus draw of the fused draft -> verification path, from the
// residual mode's tile sums.  One workgroup of four wavefronts per request
// the acceptance scan left without an error flag (a flagged request's outputs
// are already written):
//   tile choice   thread t holds tile sums [t per, (t + 1) per); fp64 prefix
//                 (thread runs, then a deterministic block scan) and total Z;
//                 the first tile whose cumulative sum, rounded to binary32,
//                 exceeds fp32(u' * fp32(Z)), else the last tile with weight
//                 (inverse CDF in ascending token order, as the oracle's);
//   the tile      its 64 weights with the residual epilogue's arithmetic:
//                 the draft logits rebuilt by MFMA as the Markov draw does
//                 (same Wt rows, same k order, same base add), the target
//                 logits read back, both weighed by resid_weight;
//   the token     wavefront 0: fp64 prefix of the weights from the mass
//                 before the tile, the first token past the threshold, else
//                 the tile's last token with weight.
// A residual whose mass rounds to zero (Z <= 0 after a rejection; in exact
// arithmetic a rejection implies p != q) falls back to the p row: the
// workgroup sums p's tile weights itself (rare; one pass over the row) and
// draws from them, flagging SV_FLAG_RESID_ZERO.
// ---------------------------------------------------------------------------
struct ResidSel {
    double Z;       // total weight
    float tf;       // fp32(u * fp32(Z))
    double tbase;   // cumulative weight before the chosen tile
    int ts;         // chosen tile
    int fallback;   // no cumulative weight exceeded tf: the last token with weight
};

// Tile choice over the tile sums ts[0 .. ntile) (global or LDS) by the whole
// workgroup; every thread returns the same result, false when no tile has
// weight.
__device__ bool choose_resid_tile(const float *ts_sum, int ntile, float u, DrawLDS &L, ResidSel &st)
{
    const int t = threadIdx.x, lane = t & 63, wid = t >> 6;
    const int per = (ntile + kDrawThreads - 1) / kDrawThreads;
    const int t0 = t * per;
    float wt[kDrawTilesPerThread];
    double loc = 0.0;
#pragma unroll
    for (int q = 0; q < kDrawTilesPerThread; ++q) {
        wt[q] = (q < per && t0 + q < ntile) ? ts_sum[t0 + q] : 0.0f;
        loc += (double)wt[q];
    }
    double Z;
    const double excl = svk::block_exclusive_scan_d<kDrawThreads>(loc, L.scan, &Z);
    const float tf = __fmul_rn(u, (float)Z);
    int first = 0x7FFFFFFF, last = -1;
    double firstb = 0.0, lastb = 0.0;
    {
        double run = excl;
#pragma unroll
        for (int q = 0; q < kDrawTilesPerThread; ++q) {
            if (wt[q] > 0.0f) {
                const double before = run;
                run += (double)wt[q];
                last = t0 + q;
                lastb = before;
                if (first == 0x7FFFFFFF && (float)run > tf) {
                    first = t0 + q;
                    firstb = before;
                }
            }
        }
    }
    {
        const uint64_t hasf = __ballot(first != 0x7FFFFFFF), hasl = __ballot(last >= 0);
        const int lf = hasf ? __builtin_ctzll(hasf) : 0;
        const int ll = hasl ? 63 - __builtin_clzll(hasl) : 0;
        const int fw = __shfl(first, lf, 64), lw = __shfl(last, ll, 64);
        const double fbw = __shfl(firstb, lf, 64), lbw = __shfl(lastb, ll, 64);
        if (lane == 0) {
            L.wfirst[wid] = hasf ? fw : 0x7FFFFFFF;
            L.wfirstb[wid] = fbw;
            L.wlast[wid] = hasl ? lw : -1;
            L.wlastb[wid] = lbw;
        }
    }
    __syncthreads();
    int ts = 0x7FFFFFFF, tl = -1;
    double tb = 0.0, tlb = 0.0;
#pragma unroll
    for (int w = 0; w < kDrawWaves; ++w) {
        if (ts == 0x7FFFFFFF && L.wfirst[w] != 0x7FFFFFFF) {
            ts = L.wfirst[w];
            tb = L.wfirstb[w];
        }
        if (L.wlast[w] >= 0) {
            tl = L.wlast[w];
            tlb = L.wlastb[w];
        }
    }
    __syncthreads();   // L is reused by a second choice
    const bool fallback = ts == 0x7FFFFFFF;
    st.Z = Z;
    st.tf = tf;
    st.tbase = fallback ? tlb : tb;
    st.ts = fallback ? tl : ts;
    st.fallback = fallback;
    return tl >= 0 && Z > 0.0;
}

// The sum of p's tile weights 2^(xp c - lp2) of every tile into out[] (LDS),
// by the whole workgroup: wavefront w takes tiles w, w + 4, ...; lane l
// weighs token l of the tile.
template <int PES>
__device__ void p_tile_sums(const char *prow, float lp2, float c, int64_t V, int ntile, float *out)
{
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    for (int tl = wid; tl < ntile; tl += kDrawWaves) {
        const int64_t c0 = (int64_t)tl * TN;
        const int64_t n = c0 + lane;
        float w = n < V ? resid_weight(svk::load_logit<PES>(prow, n), 0.0f, 1, 1.0f, lp2, 0.0f, c) : 0.0f;
        w = svk::wave_sum(w);
        if (lane == 0) out[tl] = w;
    }
}

template <int R, int PES>
__global__ __launch_bounds__(kDrawThreads) void k_markov_resid_draw(svh::MarkovArgs a, svh::VerifyArgs v,
                                                                    const svh::ReqG *__restrict__ req,
                                                                    const float *__restrict__ tsum, int ntile,
                                                                    uint32_t *__restrict__ errword)
{
    constexpr int KS = R / 32;
    constexpr int VBW = NVB / kDrawWaves;   // 16-row blocks per wavefront
    __shared__ DrawLDS L;
    __shared__ float wtile[TN];                  // the chosen tile's weights
    __shared__ float alt[svh::kMarkovMaxTiles];  // p's tile sums (zero-residual fallback)
    const int b = blockIdx.x;
    const int t = threadIdx.x, lane = t & 63, wid = t >> 6;
    const int li = lane & 15, lg = lane >> 4;
    const svh::ReqG r = req[b];
    if (r.flags) return;   // the acceptance scan wrote the request's outputs
    const int G1 = a.gamma + 1;
    const int k = r.tau + 1;   // the draft position of the correction row
    const char *prow = (const char *)v.p + ((int64_t)b * G1 + r.tau) * a.V * PES;
    bf16x8 ufr[KS];
    head_fragments<R>(a, k, b, lg, r.mode == 0, ufr);   // requested before the tile choice

    int mode = r.mode;
    float wmul = r.wmul;
    uint32_t flags = 0;
    ResidSel st;
    bool ok = choose_resid_tile(tsum + (int64_t)b * ntile, ntile, r.u2, L, st);
    if (!ok && mode == 0) {
        flags |= SV_FLAG_RESID_ZERO;
        mode = 1;
        wmul = 1.0f;
        p_tile_sums<PES>(prow, r.lp2, a.c, a.V, ntile, alt);
        __syncthreads();
        ok = choose_resid_tile(alt, ntile, r.u2, L, st);
    }
    int32_t y = -1;
    if (ok) {
        const int64_t c0 = (int64_t)st.ts * TN;
        const int ncols = (int)((a.V - c0) < TN ? (a.V - c0) : TN);
        if (mode == 0) {
            bf16x8 afr[VBW][KS];
#pragma unroll
            for (int vb = 0; vb < VBW; ++vb) {
                const int64_t n = c0 + 16 * (VBW * wid + vb) + li;
                const uint16_t *wrow = a.W + (n < a.V ? n : a.V - 1) * R + 8 * lg;
#pragma unroll
                for (int s = 0; s < KS; ++s) afr[vb][s] = *(const bf16x8 *)(wrow + 32 * s);
            }
            // base and target logits of the lane's outputs, requested with
            // the A rows (an in-row address for every column)
            const uint16_t *brow = a.base + ((int64_t)b * a.gamma + (k - 1)) * a.V + c0;
            uint32_t bbits[VBW][4];
            float xp[VBW][4];
#pragma unroll
            for (int vb = 0; vb < VBW; ++vb)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int col = 16 * (VBW * wid + vb) + 4 * lg + q;
                    const int cc = col < ncols ? col : 0;
                    bbits[vb][q] = brow[cc];
                    xp[vb][q] = svk::load_logit<PES>(prow, c0 + cc);
                }
#pragma unroll
            for (int vb = 0; vb < VBW; ++vb) {
                f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < KS; ++s)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr[vb][s], ufr[s], acc, 0, 0, 0);
                if (li == 0) {   // D[4 lg + q][0]: vocabulary row 16 vb + 4 lg + q of the tile
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int col = 16 * (VBW * wid + vb) + 4 * lg + q;
                        const float z = acc[q] + __uint_as_float(bbits[vb][q] << 16);
                        wtile[col] = col < ncols ? resid_weight(xp[vb][q], z, 0, wmul, r.lp2, r.lq2, a.c) : 0.0f;
                    }
                }
            }
        } else if (t < TN) {
            wtile[t] = t < ncols ? resid_weight(svk::load_logit<PES>(prow, c0 + t), 0.0f, 1, wmul, r.lp2, r.lq2, a.c)
                                 : 0.0f;
        }
        svk::lds_barrier();
        if (wid == 0) {
            const int j0 = lane;
            const float w0 = wtile[j0];
            const double pincl = svk::wave_inclusive_scan_d((double)w0);
            const double pexcl = pincl - (double)w0;
            int yb = 0x7FFFFFFF, yl = -1;
            if (w0 > 0.0f) {
                yl = j0;
                if (!st.fallback && (float)(st.tbase + pexcl + (double)w0) > st.tf) yb = j0;
            }
            const int ybest = wave_min_i(yb);
            const int ylast = wave_max_i(yl);
            const int j = ybest != 0x7FFFFFFF ? ybest : ylast;
            y = j >= 0 ? (int32_t)(c0 + j) : -1;
        }
    }
    if (wid != 0) return;
    if (y < 0) flags |= SV_FLAG_BAD_ROW;   // unreachable for a valid row: p sums to 1
    // x_1 .. x_tau, the drawn token, then -1 (all -1 and length -1 if none)
    const int64_t ob = (int64_t)b * G1;
    for (int j = lane; j < G1; j += 64)
        v.out_tokens[ob + j] =
            y < 0 ? -1 : (j < r.tau ? a.draft[(int64_t)b * a.gamma + j] : (j == r.tau ? y : -1));
    if (lane == 0) {
        v.accepted_len[b] = y < 0 ? -1 : r.tau;
        if (v.diag.flags) v.diag.flags[b] = flags;
        if (v.diag.resid_mass) v.diag.resid_mass[b] = (float)st.Z;
        if (flags) atomicOr(errword, flags);
    }
}

// Every base-logit row starts on a 16-byte boundary (the loaders copy it with
// 16-byte direct loads); otherwise they copy element by element.
inline int base_rows_aligned(const svh::MarkovArgs &a)
{
    return (a.V % 8 == 0) && ((((uintptr_t)a.base) & 15) == 0);
}

template <int R>
hipError_t launch_positions(sv_ctx *ctx, const svh::MarkovArgs &args, hipStream_t s)
{
    // The Markov head stages its operand rows too: a small kernel copies
    // U[x_0] of every request into the state buffer (the RNN head's, unused
    // here) before position 1, each draw then leaves U[x_k] there, and the
    // contraction's loaders copy those rows as they do the RNN states.
    svh::MarkovArgs a = args;
    if (!a.A) a.hstate = ctx->ws.rnn_h;
    const int ntile = ctx->ntile;
    const int gy = (a.B + MC - 1) / MC;
    int gx = ctx->num_cu / gy;   // one workgroup per CU (its tile ring fills most of the LDS)
    gx = gx < 1 ? 1 : (gx > ntile ? ntile : gx);
    // z rows of position k: the caller's q_logits [B, gamma, V], else a
    // workspace row per request
    const int64_t zstride = a.q_logits ? (int64_t)a.gamma * a.V : a.V;
    const int vec = base_rows_aligned(a);
    const int zvec = (a.V % 4 == 0) && ((((uintptr_t)(a.q_logits ? a.q_logits : ctx->ws.mk_q)) & 15) == 0);
    // riding target-row chunks: an even share per draw
    const int64_t ride_per = a.ride.items > 0 ? (a.ride.items + a.gamma - 1) / a.gamma : 0;
    if (a.A)
        hipLaunchKernelGGL(k_rnn_first_state, dim3(a.B), dim3(a.R < 256 ? a.R : 256), 0, s, a);
    else
        hipLaunchKernelGGL((k_markov_first_rows<R>), dim3(a.B), dim3(64), 0, s, a);
    for (int k = 1; k <= a.gamma; ++k) {
        const int64_t r0 = ride_per * (k - 1);
        const int64_t rn = a.ride.items - r0 < ride_per ? (a.ride.items - r0 > 0 ? a.ride.items - r0 : 0) : ride_per;
        float *zk = a.fused ? nullptr : (a.q_logits ? a.q_logits + (int64_t)(k - 1) * a.V : ctx->ws.mk_q);
        int slot = svh::prof_begin(ctx, s, SV_KERNEL_MARKOV_GEMM);
        hipLaunchKernelGGL((k_markov_gemm<R, 0, true>), dim3(gx, gy), dim3(NTG), 0, s, a, k,
                           (const svh::ReqG *)nullptr, zk, zstride, ctx->ws.mk_part, ntile, vec, zvec,
                           ResidArgs{nullptr, nullptr}, 0);
        svh::prof_end(ctx, s, slot);
        slot = svh::prof_begin(ctx, s, SV_KERNEL_MARKOV_SELECT);
        const int64_t cap = (int64_t)SV_MARKOV_RIDE_WGS_PER_CU * ctx->num_cu;
        const int64_t nride = rn < cap ? rn : cap;
        if (nride > 0)
            hipLaunchKernelGGL((k_markov_draw<R, true>), dim3((unsigned)(a.B + nride)), dim3(kDrawThreads), 0, s, a,
                               k, (const float *)zk, zstride, (const float2 *)ctx->ws.mk_part, ntile, ctx->ws.errword,
                               r0, rn);
        else
            hipLaunchKernelGGL((k_markov_draw<R, false>), dim3((unsigned)a.B), dim3(kDrawThreads), 0, s, a, k,
                               (const float *)zk, zstride, (const float2 *)ctx->ws.mk_part, ntile, ctx->ws.errword,
                               (int64_t)0, (int64_t)0);
        svh::prof_end(ctx, s, slot);
    }
    return hipGetLastError();
}

template <int R, int PES>
hipError_t launch_resid(sv_ctx *ctx, const svh::MarkovArgs &a, const svh::VerifyArgs &v, const svh::ReqG *req,
                        hipStream_t s)
{
    const int ntile = ctx->ntile;
    const int gy = (a.B + MC - 1) / MC;
    int gx = ctx->num_cu / gy;
    gx = gx < 1 ? 1 : (gx > ntile ? ntile : gx);
    const int vec = base_rows_aligned(a);
    const int pvec = (a.V % 4 == 0) && ((((uintptr_t)v.p) & (4 * PES - 1)) == 0);
    // the draft's tile pairs are consumed: their buffer holds the tile sums
    float *tsum = (float *)ctx->ws.mk_part;
    int slot = svh::prof_begin(ctx, s, SV_KERNEL_MARKOV_REBUILD);
    hipLaunchKernelGGL((k_markov_gemm<R, PES, false>), dim3(gx, gy), dim3(NTG), 0, s, a, 0, req, (float *)nullptr, a.V,
                       (float2 *)nullptr, ntile, vec, 0, ResidArgs{v.p, tsum}, pvec);
    svh::prof_end(ctx, s, slot);
    slot = svh::prof_begin(ctx, s, SV_KERNEL_SELECT);
    hipLaunchKernelGGL((k_markov_resid_draw<R, PES>), dim3(a.B), dim3(kDrawThreads), 0, s, a, v, req,
                       (const float *)tsum, ntile, ctx->ws.errword);
    svh::prof_end(ctx, s, slot);
    return hipGetLastError();
}

template <int PES>
hipError_t launch_resid_rank(sv_ctx *ctx, const svh::MarkovArgs &a, const svh::VerifyArgs &v, const svh::ReqG *req,
                             hipStream_t s)
{
    switch (a.R) {
    case 32: return launch_resid<32, PES>(ctx, a, v, req, s);
    case 64: return launch_resid<64, PES>(ctx, a, v, req, s);
    case 128: return launch_resid<128, PES>(ctx, a, v, req, s);
    case 256: return launch_resid<256, PES>(ctx, a, v, req, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

namespace svh {

hipError_t launch_markov_resid(sv_ctx *ctx, const MarkovArgs &a, const VerifyArgs &v, const ReqG *req,
                               hipStream_t s)
{
    if (a.B <= 0) return hipSuccess;
    return v.p_esize == 2 ? launch_resid_rank<2>(ctx, a, v, req, s) : launch_resid_rank<4>(ctx, a, v, req, s);
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
