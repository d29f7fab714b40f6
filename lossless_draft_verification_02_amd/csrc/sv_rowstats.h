// sv_rowstats.h -- per-thread softmax statistics of a run of logits, shared
// by the row-statistics pass, the single-launch verification of small
// problems and the target-row chunks that ride in the Markov draws.
#pragma once

#include "sv_device.h"

namespace svk {

// A chunk [e0, e1) of one row split into a 16-byte aligned body of nvec
// vectors starting at element a0, and scalar elements before (head) and
// after (tail) it.
template <int ESIZE>
struct ChunkPlan {
    const char *rowptr;
    const u32x4 *vec;
    int64_t e0, a0, a1, e1, nvec;
};

template <int ESIZE>
__device__ __forceinline__ ChunkPlan<ESIZE> chunk_plan(const char *__restrict__ rowptr, int64_t e0, int64_t e1)
{
    constexpr int EPV = 16 / ESIZE;   // elements per 16-byte vector
    const uintptr_t addr0 = (uintptr_t)(rowptr + e0 * ESIZE);
    int64_t head = (int64_t)(((16 - (addr0 & 15)) & 15) / ESIZE);
    if (head > e1 - e0) head = e1 - e0;
    ChunkPlan<ESIZE> pl;
    pl.rowptr = rowptr;
    pl.e0 = e0;
    pl.e1 = e1;
    pl.a0 = e0 + head;
    pl.nvec = (e1 - pl.a0) / EPV;
    pl.a1 = pl.a0 + pl.nvec * EPV;
    pl.vec = (const u32x4 *)(rowptr + pl.a0 * ESIZE);
    return pl;
}

// One batch of NB vectors of the body, v0 + j NT for j < NB; past the body
// the vectors read as -inf.
template <int ESIZE, int NB, int NT>
__device__ __forceinline__ void load_batch(const ChunkPlan<ESIZE> &pl, int64_t v0, bool nontemporal, u32x4 *raw)
{
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        const int64_t idx = v0 + (int64_t)j * NT;
        if (nontemporal)
            raw[j] = idx < pl.nvec ? __builtin_nontemporal_load(pl.vec + idx) : svk::neg_inf_vec<ESIZE>();
        else
            raw[j] = idx < pl.nvec ? pl.vec[idx] : svk::neg_inf_vec<ESIZE>();
    }
}

// Running statistics of one thread: the max in raw units and scaled by c,
// and the sum of exp2(x c - mref).
struct RunStats {
    float mref, mraw, s;
};

__device__ __forceinline__ RunStats run_start()
{
    return RunStats{svk::neg_inf(), svk::neg_inf(), 0.0f};
}

// Folds one loaded batch into the running statistics.
//
// The reference ref = round(max * c) must be the same rounded value in every
// use: the terms are exp2(x * c - ref) (one fused multiply-add) and an
// earlier partial sum is rescaled by exp2(ref_old - ref).  Contracting the
// product into the rescale's subtraction would use the unrounded max * c
// there and scale the whole partial sum by the product's rounding error; no
// contraction here.
template <int ESIZE, int NB>
__device__ __forceinline__ void fold_batch(const u32x4 *raw, float c, RunStats &r)
{
#pragma clang fp contract(off)
    constexpr int EPV = 16 / ESIZE;
    float x[NB * EPV];
#pragma unroll
    for (int j = 0; j < NB; ++j) svk::widen<ESIZE>(raw[j], x + j * EPV);
    float bm = x[0];
#pragma unroll
    for (int k = 1; k < NB * EPV; ++k) bm = fmaxf(bm, x[k]);
    const float nm = fmaxf(r.mraw, bm);
    if (nm == svk::neg_inf()) {
        // everything so far is -inf; only a NaN can still matter
#pragma unroll
        for (int k = 0; k < NB * EPV; ++k)
            if (x[k] != x[k]) r.s = x[k];
        return;
    }
    const float ref = nm * c;
    r.s *= svk::fast_exp2(r.mref - ref);
    float acc = 0.0f;
#pragma unroll
    for (int k = 0; k < NB * EPV; ++k) acc += svk::fast_exp2(__builtin_fmaf(x[k], c, -ref));
    r.s += acc;
    r.mraw = nm;
    r.mref = ref;
}

// Adds this thread's scalar element of the head [e0, a0) and tail [a1, e1)
// (fewer than 2 * EPV elements in all) and returns the thread's (m, s).
template <int ESIZE>
__device__ __forceinline__ MS run_finish(const ChunkPlan<ESIZE> &pl, float c, int tid, const RunStats &r)
{
#pragma clang fp contract(off)
    float mref = r.mref, s = r.s;
    const int64_t nhead = pl.a0 - pl.e0;
    const int64_t nscalar = nhead + (pl.e1 - pl.a1);
    if ((int64_t)tid < nscalar) {
        const int64_t e = (int64_t)tid < nhead ? pl.e0 + tid : pl.a1 + ((int64_t)tid - nhead);
        const float x = svk::load_logit<ESIZE>(pl.rowptr, e);
        MS one;
        if (x == svk::neg_inf()) {
            one = {svk::neg_inf(), 0.0f};
        } else if (x != x || x == svk::pos_inf()) {
            one = {svk::pos_inf(), __builtin_nanf("")};
        } else {
            one = {x * c, 1.0f};
        }
        const MS a = svk::ms_merge(MS{mref, s}, one);
        mref = a.m;
        s = a.s;
    }
    return MS{mref, s};
}

// This thread's (m, s) over its share of elements [e0, e1) of one row, the
// share of thread `tid` of NT cooperating threads (a workgroup or a
// wavefront): batches of NB 16-byte vectors, each folded in as it lands,
// then the scalar head and tail.
template <int ESIZE, int NB, int NT>
__device__ __forceinline__ MS thread_stats(const char *__restrict__ rowptr, int64_t e0, int64_t e1, float c,
                                           bool nontemporal, int tid)
{
    const ChunkPlan<ESIZE> pl = chunk_plan<ESIZE>(rowptr, e0, e1);
    RunStats r = run_start();
    for (int64_t v0 = tid; v0 < pl.nvec; v0 += (int64_t)NT * NB) {
        u32x4 raw[NB];
        load_batch<ESIZE, NB, NT>(pl, v0, nontemporal, raw);
        fold_batch<ESIZE, NB>(raw, c, r);
    }
    return run_finish<ESIZE>(pl, c, tid, r);
}

}  // namespace svk
