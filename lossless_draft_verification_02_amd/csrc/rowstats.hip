// rowstats.hip -- single-pass softmax statistics of every verified logit row.
//
// The acceptance ratio p(x)/q(x) and the residual max(p - q, 0) are defined on
// normalised distributions ("Speculative Decoding: The Same Distribution,
// Twice as Fast", section 4 "The rule that makes it exact"), so every target
// and draft row a request verifies needs its log-sum-exp over the whole
// vocabulary.  This kernel streams each row once from HBM and writes, per row
// chunk, the pair (m, s) = (max x*c, sum exp2(x*c - m)) with c = log2(e)/T.
//
// Work decomposition: one 256-thread workgroup per (row, chunk); a chunk is
// `chunk1` elements (a multiple of 8).  Threads read 16-byte vectors in a
// strided, coalesced pattern, NB vectors in flight per thread, and fold each
// batch into a running (m, s): one max, one fma, one exp2 and one add per
// element, plus one rescale per batch.  Unaligned row starts (odd V with bf16)
// are handled by a scalar head and tail.  Rows a request does not verify
// (beyond verify_len) are never read: with per-request lengths on the device,
// a fixed grid of workgroups walks a compacted list of the verified items
// instead of dispatching a workgroup per item of the full [B, gamma] shape.
#include "sv_device.h"
#include "sv_internal.h"
#include "sv_rowstats.h"

namespace {

using svk::MS;
using svk::u32x4;
using svk::thread_stats;

// (m, s) of elements [e0, e1) of one row by the whole workgroup; valid in thread 0.
template <int ESIZE, int NB>
__device__ __forceinline__ MS chunk_stats(const char *__restrict__ rowptr, int64_t e0, int64_t e1, float c,
                                          bool nontemporal, MS *red)
{
    constexpr int NT = svh::kRowstatsThreads;
    return svk::block_merge<NT>(thread_stats<ESIZE, NB, NT>(rowptr, e0, e1, c, nontemporal, threadIdx.x), red);
}

// Statistics of chunk `chunk` of row i of request b (a p row when is_p,
// else a q row) into part[], by the whole workgroup (WAVE false) or by one
// wavefront on its own (WAVE true: shuffles only, no LDS, no barrier).  A
// request has np p rows and nq q rows (gamma + 1 and gamma for a draft).
template <int PES, int QES, int NB, bool WAVE>
__device__ __forceinline__ void rowstats_chunk(const void *__restrict__ p, const void *__restrict__ q, int B,
                                               int np, int nq, int b, int i, bool is_p, int chunk, int64_t V,
                                               int nch1, int64_t chunk1, float c, float2 *__restrict__ part, MS *red)
{
    const int64_t e0 = (int64_t)chunk * chunk1;
    const int64_t e1 = e0 + chunk1 < V ? e0 + chunk1 : V;
    const bool nontemporal = SV_ROWSTATS_NT_LOADS;
    int64_t grow;   // row index in the statistics array: all p rows, then all q rows
    const char *row;
    int esize;
    if (is_p) {
        grow = (int64_t)b * np + i;
        row = (const char *)p + grow * V * PES;
        esize = PES;
    } else {
        const int64_t qr = (int64_t)b * nq + i;
        grow = (int64_t)B * np + qr;
        row = (const char *)q + qr * V * QES;
        esize = QES;
    }
    MS tot;
    if constexpr (WAVE) {
        const int lane = threadIdx.x & (svk::kWave - 1);
        if constexpr (PES == QES)
            tot = thread_stats<PES, NB, svk::kWave>(row, e0, e1, c, nontemporal, lane);
        else
            tot = esize == PES ? thread_stats<PES, NB, svk::kWave>(row, e0, e1, c, nontemporal, lane)
                               : thread_stats<QES, NB, svk::kWave>(row, e0, e1, c, nontemporal, lane);
        tot = svk::wave_merge(tot);
        if (lane == 0) part[grow * nch1 + chunk] = make_float2(tot.m, tot.s);
    } else {
        if constexpr (PES == QES)
            tot = chunk_stats<PES, NB>(row, e0, e1, c, nontemporal, red);
        else
            tot = esize == PES ? chunk_stats<PES, NB>(row, e0, e1, c, nontemporal, red)
                               : chunk_stats<QES, NB>(row, e0, e1, c, nontemporal, red);
        if (threadIdx.x == 0) part[grow * nch1 + chunk] = make_float2(tot.m, tot.s);
    }
}

// One workgroup per (row, chunk) item of requests [b0, b0 + nb): p rows
// first (np per request), then q rows (nq per request).  Without verify
// lengths every row is read and the grid is exactly the work; with them
// (draft layout, np = gamma + 1, nq = gamma), rows past a request's length
// return at once.
template <int PES, int QES, int NB>
__global__ __launch_bounds__(svh::kRowstatsThreads) void k_rowstats(
    const void *__restrict__ p, const void *__restrict__ q, const int32_t *__restrict__ verify_len, int B,
    int np, int nq, int b0, int nb, int64_t V, int nch1, int64_t chunk1, float c, float2 *__restrict__ part)
{
    __shared__ MS red[svh::kRowstatsThreads / svk::kWave];
    const int64_t slot = blockIdx.x / nch1;
    const int chunk = (int)(blockIdx.x - slot * nch1);
    const int64_t lrows_p = (int64_t)nb * np;
    int bl, i;
    const bool is_p = slot < lrows_p;
    if (is_p) {
        bl = (int)(slot / np);
        i = (int)(slot - (int64_t)bl * np);
    } else {
        const int64_t r = slot - lrows_p;
        bl = (int)(r / nq);
        i = (int)(r - (int64_t)bl * nq);
    }
    if (verify_len) {
        const int L = verify_len[b0 + bl];
        if (L < 0 || L > nq || (is_p ? i > L : i >= L)) return;
    }
    rowstats_chunk<PES, QES, NB, false>(p, q, B, np, nq, b0 + bl, i, is_p, chunk, V, nch1, chunk1, c, part, red);
}

// Calls with per-request verify lengths L_b (on the device): only rows
// 0..L_b of p and 0..L_b-1 of q are read.  Every workgroup first lays out in
// LDS the lengths and the running count of verified items (rows x chunks)
// per request, then takes every gridDim.x-th verified item, so the work is
// balanced and an unverified row costs nothing.  A length outside [0, gamma]
// verifies no row (the request is flagged downstream).  After the layout
// each wavefront takes whole (row, chunk) items on its own, so no barrier
// stalls the memory pipeline between items.
template <int PES, int QES, int NB>
__global__ __launch_bounds__(svh::kRowstatsThreads) void k_rowstats_compact(
    const void *__restrict__ p, const void *__restrict__ q, const int32_t *__restrict__ verify_len, int B,
    int gamma, int b0, int nb, int64_t V, int nch1, int64_t chunk1, float c, float2 *__restrict__ part)
{
    constexpr int NT = svh::kRowstatsThreads;
    __shared__ int wsum[NT / svk::kWave];
    extern __shared__ int dyn[];
    int *Ls = dyn;              // [nb] verify lengths, -1 for an invalid one
    int *pre = dyn + nb;        // [nb + 1] first item of each request; pre[nb] = total

    // per-request item counts (rows x chunks), thread t owning a contiguous run
    const int t = threadIdx.x;
    const int per = (nb + NT - 1) / NT;
    const int r0 = t * per, r1 = r0 + per < nb ? r0 + per : nb;
    int loc = 0;
    for (int bl = r0; bl < r1; ++bl) {
        int L = verify_len[b0 + bl];
        L = (L >= 0 && L <= gamma) ? L : -1;
        Ls[bl] = L;
        const int cnt = L >= 0 ? (2 * L + 1) * nch1 : 0;
        pre[bl] = cnt;
        loc += cnt;
    }
    // exclusive block scan of the per-thread totals
    const int lane = t & (svk::kWave - 1), wid = t / svk::kWave;
    int incl = loc;
#pragma unroll
    for (int o = 1; o < svk::kWave; o <<= 1) {
        const int y = __shfl_up(incl, o, svk::kWave);
        if (lane >= o) incl += y;
    }
    if (lane == svk::kWave - 1) wsum[wid] = incl;
    __syncthreads();
    int run = incl - loc;
    for (int w = 0; w < wid; ++w) run += wsum[w];
    for (int bl = r0; bl < r1; ++bl) {
        const int cnt = pre[bl];
        pre[bl] = run;
        run += cnt;
    }
    if (t == NT - 1) {
        int tot = 0;
        for (int w = 0; w < NT / svk::kWave; ++w) tot += wsum[w];
        pre[nb] = tot;
    }
    __syncthreads();

    // from here on every wavefront works alone: items are taken per wavefront
    const int total = pre[nb];
    const int nw = (int)gridDim.x * (NT / svk::kWave);
    int lo = 0;
    for (int item = (int)blockIdx.x * (NT / svk::kWave) + wid; item < total; item += nw) {
        // request holding the item: the largest bl >= lo with pre[bl] <= item
        int hi = nb - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (pre[mid] <= item) lo = mid;
            else hi = mid - 1;
        }
        const int r = item - pre[lo];
        const int row = r / nch1, chunk = r - row * nch1;
        const int L = Ls[lo];
        const bool is_p = row <= L;
        rowstats_chunk<PES, QES, NB, true>(p, q, B, gamma + 1, gamma, b0 + lo, is_p ? row : row - (L + 1), is_p,
                                           chunk, V, nch1, chunk1, c, part, nullptr);
    }
}

template <int PES, int QES>
void launch_typed(sv_ctx *ctx, const svh::VerifyArgs &a, hipStream_t s, int64_t items, int np, int nq)
{
    constexpr int NB = svh::kRowstatsNB;
    const bool compact = a.verify_len && a.nb <= svh::kRowstatsCompactMaxReq && items <= 0x7FFFFFFF;
    if (compact) {
        const int64_t cap = (int64_t)svh::kRowstatsCompactWGsPerCU * ctx->num_cu;
        const int64_t grid = items < cap ? items : cap;
        const size_t lds = (size_t)(2 * a.nb + 1) * sizeof(int);
        hipLaunchKernelGGL((k_rowstats_compact<PES, QES, svh::kRowstatsCompactNB>), dim3((unsigned)grid),
                           dim3(svh::kRowstatsThreads), lds,
                           s, a.p, a.q, a.verify_len, a.B, a.gamma, a.b0, a.nb, a.V, ctx->nch1, ctx->chunk1, a.c,
                           ctx->ws.part);
    } else {
        hipLaunchKernelGGL((k_rowstats<PES, QES, NB>), dim3((unsigned)items), dim3(svh::kRowstatsThreads), 0, s,
                           a.p, a.q, a.verify_len, a.B, np, nq, a.b0, a.nb, a.V, ctx->nch1, ctx->chunk1, a.c,
                           ctx->ws.part);
    }
}

}  // namespace

namespace svh {

hipError_t launch_rowstats(sv_ctx *ctx, const VerifyArgs &a, hipStream_t s)
{
    // p rows, then q rows unless the q statistics come from the Markov sampler
    const int np = a.np_rows ? a.np_rows : a.gamma + 1;
    const int nq = a.np_rows ? a.nq_rows : a.gamma;
    const int64_t rows = (int64_t)a.nb * np + (a.q_lse2 ? 0 : (int64_t)a.nb * nq);
    const int64_t grid = rows * ctx->nch1;
    if (grid <= 0) return hipSuccess;
    const int slot = prof_begin(ctx, s, SV_KERNEL_ROWSTATS);
    if (a.p_esize == 2 && a.q_esize == 2) launch_typed<2, 2>(ctx, a, s, grid, np, nq);
    else if (a.p_esize == 2) launch_typed<2, 4>(ctx, a, s, grid, np, nq);
    else if (a.q_esize == 2) launch_typed<4, 2>(ctx, a, s, grid, np, nq);
    else launch_typed<4, 4>(ctx, a, s, grid, np, nq);
    const hipError_t e = hipGetLastError();
    prof_end(ctx, s, slot);
    return e;
}

}  // namespace svh
