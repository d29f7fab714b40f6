// sv_rowstats.h -- per-thread softmax statistics of a run of logits, shared
// by the row-statistics pass and the single-launch verification of small
// problems.
#pragma once

#include "sv_device.h"

namespace svk {

// This thread's (m, s) over its share of elements [e0, e1) of one row, the
// share of thread `tid` of NT cooperating threads (a workgroup or a wavefront).
template <int ESIZE, int NB, int NT>
__device__ __forceinline__ MS thread_stats(const char *__restrict__ rowptr, int64_t e0, int64_t e1, float c,
                                           bool nontemporal, int tid)
{
    // The reference ref = round(max * c) must be the same rounded value in
    // every use: the terms are exp2(x * c - ref) (one fused multiply-add) and
    // an earlier partial sum is rescaled by exp2(ref_old - ref).  Contracting
    // the product into the rescale's subtraction would use the unrounded
    // max * c there and scale the whole partial sum by the product's rounding
    // error; no contraction here.
#pragma clang fp contract(off)
    constexpr int EPV = 16 / ESIZE;   // elements per 16-byte vector

    // 16-byte aligned body [a0, a1) inside [e0, e1)
    const uintptr_t addr0 = (uintptr_t)(rowptr + e0 * ESIZE);
    int64_t head = (int64_t)(((16 - (addr0 & 15)) & 15) / ESIZE);
    if (head > e1 - e0) head = e1 - e0;
    const int64_t a0 = e0 + head;
    const int64_t nvec = (e1 - a0) / EPV;
    const int64_t a1 = a0 + nvec * EPV;
    const u32x4 *vec = (const u32x4 *)(rowptr + a0 * ESIZE);

    float mref = svk::neg_inf();   // running max, scaled by c
    float mraw = svk::neg_inf();   // running max, raw units
    float s = 0.0f;

    for (int64_t v0 = tid; v0 < nvec; v0 += (int64_t)NT * NB) {
        u32x4 raw[NB];
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const int64_t idx = v0 + (int64_t)j * NT;
            if (nontemporal)
                raw[j] = idx < nvec ? __builtin_nontemporal_load(vec + idx) : svk::neg_inf_vec<ESIZE>();
            else
                raw[j] = idx < nvec ? vec[idx] : svk::neg_inf_vec<ESIZE>();
        }
        float x[NB * EPV];
#pragma unroll
        for (int j = 0; j < NB; ++j) svk::widen<ESIZE>(raw[j], x + j * EPV);
        float bm = x[0];
#pragma unroll
        for (int k = 1; k < NB * EPV; ++k) bm = fmaxf(bm, x[k]);
        const float nm = fmaxf(mraw, bm);
        if (nm == svk::neg_inf()) {
            // everything so far is -inf; only a NaN can still matter
#pragma unroll
            for (int k = 0; k < NB * EPV; ++k)
                if (x[k] != x[k]) s = x[k];
            continue;
        }
        const float ref = nm * c;
        s *= svk::fast_exp2(mref - ref);
        float acc = 0.0f;
#pragma unroll
        for (int k = 0; k < NB * EPV; ++k) acc += svk::fast_exp2(__builtin_fmaf(x[k], c, -ref));
        s += acc;
        mraw = nm;
        mref = ref;
    }

    // scalar head [e0, a0) and tail [a1, e1): fewer than 2 * EPV elements
    const int64_t nhead = a0 - e0;
    const int64_t nscalar = nhead + (e1 - a1);
    if ((int64_t)tid < nscalar) {
        const int64_t e = (int64_t)tid < nhead ? e0 + tid : a1 + ((int64_t)tid - nhead);
        const float x = svk::load_logit<ESIZE>(rowptr, e);
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

}  // namespace svk
