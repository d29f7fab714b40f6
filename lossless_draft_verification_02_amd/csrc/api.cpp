// api.cpp -- the C ABI of libspecverify: contexts, argument validation and the
// launch sequence of each call.  Declarations and contracts: spec_verify.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>

#include "spec_verify.h"
#include "sv_internal.h"

namespace {

thread_local char g_err[512] = "";

sv_status fail(sv_status st, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

sv_status ok()
{
    g_err[0] = '\0';
    return SV_OK;
}

// Makes the context's device current for the scope of a call.
struct DeviceGuard {
    int prev = -1;
    bool changed = false;
    explicit DeviceGuard(int dev)
    {
        if (hipGetDevice(&prev) == hipSuccess && prev != dev) {
            changed = hipSetDevice(dev) == hipSuccess;
        }
    }
    ~DeviceGuard()
    {
        if (changed) (void)hipSetDevice(prev);
    }
};

// The fused Markov path computes its p-row chunk statistics in extra
// workgroups of the draws' launches, which pay a fixed cost per chunk: it
// runs with chunks of about kRideChunk1 elements (or the context's, if
// longer), restored when the call returns.  Measured on MI355X (B=128,
// gamma=8, V=129,280): 0.331-0.334 ms per call at 32K-token chunks against
// 0.343-0.346 ms at the row-statistics pass's 16K and 0.344-0.348 ms at 64K.
// Longer chunks mean fewer of them per row, so the workspace sized for the
// context's geometry holds them.
constexpr int64_t kRideChunk1 = 32768;
struct RideGeometry {
    sv_ctx *ctx;
    int nch1;
    int64_t chunk1;
    explicit RideGeometry(sv_ctx *c) : ctx(c), nch1(c->nch1), chunk1(c->chunk1)
    {
        if (c->chunk1 < kRideChunk1) svh::chunk_geometry(c->vocab, kRideChunk1, &c->nch1, &c->chunk1);
    }
    ~RideGeometry()
    {
        ctx->nch1 = nch1;
        ctx->chunk1 = chunk1;
    }
};

int esize_of(sv_dtype d) { return d == SV_BF16 ? 2 : (d == SV_F32 ? 4 : 0); }

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool aligned(const void *p, size_t a) { return (((uintptr_t)p) % a) == 0; }

sv_status check_launch(hipError_t e, const char *what)
{
    if (e != hipSuccess) return fail(SV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return SV_OK;
}

// Shared validation of the verification calls.
sv_status check_verify_args(const sv_ctx *ctx, const void *p, sv_dtype pd, const void *q, sv_dtype qd,
                            const int32_t *draft, int B, int gamma, int64_t V, float T,
                            const int32_t *accepted_len, const int32_t *out_tokens, const char *fn)
{
    if (!ctx) return fail(SV_ERR_INVALID, "%s: ctx is NULL", fn);
    if (B <= 0 || B > ctx->max_batch)
        return fail(SV_ERR_INVALID, "%s: B=%d outside [1, max_batch=%d]", fn, B, ctx->max_batch);
    if (gamma < 0 || gamma > ctx->max_gamma)
        return fail(SV_ERR_INVALID, "%s: gamma=%d outside [0, max_gamma=%d]", fn, gamma, ctx->max_gamma);
    if (V != ctx->vocab)
        return fail(SV_ERR_INVALID, "%s: V=%lld differs from the context's vocab %lld", fn, (long long)V,
                    (long long)ctx->vocab);
    if (!(T > 0.0f) || !std::isfinite(T)) return fail(SV_ERR_INVALID, "%s: temperature must be finite and > 0", fn);
    if (!p || !accepted_len || !out_tokens) return fail(SV_ERR_INVALID, "%s: p, accepted_len and out_tokens are required", fn);
    if (gamma > 0 && (!q || !draft)) return fail(SV_ERR_INVALID, "%s: q and draft_tokens are required when gamma > 0", fn);
    if (esize_of(pd) == 0 || (gamma > 0 && esize_of(qd) == 0))
        return fail(SV_ERR_UNSUPPORTED, "%s: dtype must be SV_BF16 or SV_F32", fn);
    if (!aligned(p, esize_of(pd)) || (gamma > 0 && !aligned(q, esize_of(qd))))
        return fail(SV_ERR_INVALID, "%s: logits must be aligned to their element size", fn);
    return SV_OK;
}

svh::VerifyArgs make_args(const void *p, sv_dtype pd, const void *q, sv_dtype qd, const int32_t *draft,
                          const int32_t *verify_len, int B, int gamma, int64_t V, float T, uint64_t seed,
                          uint64_t offset, const float *uniforms, int32_t *accepted_len,
                          int32_t *out_tokens, const sv_diag *diag, bool block)
{
    svh::VerifyArgs a;
    a.p = p;
    a.q = q;
    a.p_esize = esize_of(pd);
    a.q_esize = gamma > 0 ? esize_of(qd) : a.p_esize;
    a.draft = draft;
    a.verify_len = verify_len;
    a.B = B;
    a.gamma = gamma;
    a.b0 = 0;
    a.nb = B;
    a.V = V;
    a.c = (float)(1.4426950408889634 / (double)T);
    a.seed = seed;
    a.offset = offset;
    a.uniforms = uniforms;
    a.accepted_len = accepted_len;
    a.out_tokens = out_tokens;
    if (diag) a.diag = *diag;
    else std::memset(&a.diag, 0, sizeof(a.diag));
    a.block = block;
    a.q_lse2 = nullptr;
    a.q_zx = nullptr;
    a.np_rows = 0;
    a.nq_rows = 0;
    return a;
}

// Row statistics, then the kernels that need them, on the caller's stream.
sv_status run_verify(sv_ctx *ctx, const svh::VerifyArgs &a, hipStream_t s,
                     hipError_t (*tail)(sv_ctx *, const svh::VerifyArgs &, hipStream_t), const char *what)
{
    sv_status st;
    if ((st = check_launch(svh::launch_rowstats(ctx, a, s), "row statistics")) != SV_OK) return st;
    return check_launch(tail(ctx, a, s), what);
}

sv_status check_markov_args(const sv_ctx *ctx, const void *base_logits, const void *U, const void *W, int R,
                            const int32_t *x0, int B, int gamma, int64_t V, float temperature,
                            const int32_t *draft_tokens, const char *fn)
{
    if (!ctx) return fail(SV_ERR_INVALID, "%s: ctx is NULL", fn);
    if (ctx->max_rank == 0) return fail(SV_ERR_INVALID, "%s: context created with max_rank 0", fn);
    if (R != ctx->max_rank) return fail(SV_ERR_INVALID, "%s: R=%d differs from max_rank %d", fn, R, ctx->max_rank);
    if (B <= 0 || B > ctx->max_batch || gamma < 1 || gamma > ctx->max_gamma)
        return fail(SV_ERR_INVALID, "%s: B=%d or gamma=%d out of range", fn, B, gamma);
    if (V != ctx->vocab) return fail(SV_ERR_INVALID, "%s: V differs from the context's vocab", fn);
    if (ctx->ntile > svh::kMarkovMaxTiles)
        return fail(SV_ERR_UNSUPPORTED, "%s: V=%lld exceeds the sampler's %d-token limit", fn, (long long)V,
                    svh::kMarkovMaxTiles * svh::kMarkovTileN);
    if (!(temperature > 0.0f) || !std::isfinite(temperature))
        return fail(SV_ERR_INVALID, "%s: temperature must be finite and > 0", fn);
    if (!base_logits || !U || !W || !x0 || !draft_tokens)
        return fail(SV_ERR_INVALID, "%s: base_logits, U, Wt, x0 and draft_tokens are required", fn);
    if (!aligned(U, 16) || !aligned(W, 16) || !aligned(base_logits, 2))
        return fail(SV_ERR_INVALID, "%s: U and Wt must be 16-byte aligned, base 2-byte aligned", fn);
    return SV_OK;
}

svh::MarkovArgs make_markov_args(const void *base_logits, const void *U, const void *W, int R, const int32_t *x0,
                                 int B, int gamma, int64_t V, float temperature, uint64_t seed, uint64_t offset,
                                 const float *uniforms, int32_t *draft_tokens, float *q_logits, float *lse_q)
{
    svh::MarkovArgs a;
    a.base = (const uint16_t *)base_logits;
    a.U = (const uint16_t *)U;
    a.W = (const uint16_t *)W;
    a.R = R;
    a.x0 = x0;
    a.B = B;
    a.gamma = gamma;
    a.V = V;
    a.c = (float)(1.4426950408889634 / (double)temperature);
    a.seed = seed;
    a.offset = offset;
    a.uniforms = uniforms;
    a.draft = draft_tokens;
    a.q_logits = q_logits;
    a.lse_q = lse_q;
    a.fused = false;
    a.lse2_out = nullptr;
    a.zx_out = nullptr;
    a.A = nullptr;
    a.hstate = nullptr;
    a.states_out = nullptr;
    a.ride = svh::RowRide{nullptr, 0, 0, 0, 0.0f, nullptr, 0};
    return a;
}

}  // namespace

namespace svh {

void chunk_geometry(int64_t vocab, int64_t target, int *nch1_out, int64_t *chunk1_out)
{
    int64_t nch1 = (vocab + target - 1) / target;
    if (nch1 < 1) nch1 = 1;
    int64_t chunk1 = (vocab + nch1 - 1) / nch1;
    chunk1 = (chunk1 + 7) / 8 * 8;
    nch1 = (vocab + chunk1 - 1) / chunk1;
    *nch1_out = (int)nch1;
    *chunk1_out = chunk1;
}

void set_geometry(sv_ctx *ctx, int64_t vocab, int64_t rows_max)
{
    // Row-statistics chunks (a multiple of 8 elements) of about
    // kTargetChunk1 elements, one batch of loads per thread of a workgroup.
    // SPECVERIFY_ROWSTATS_CHUNK (an element count) overrides the length,
    // for tuning.
    (void)rows_max;
    int64_t target = kTargetChunk1;
    if (const char *env = std::getenv("SPECVERIFY_ROWSTATS_CHUNK")) {
        const long long e = std::atoll(env);
        if (e >= 256 && e <= (1 << 22)) target = e;
    }
    chunk_geometry(vocab, target, &ctx->nch1, &ctx->chunk1);
    ctx->nseg = (int)((vocab + kSegR - 1) / kSegR);
    ctx->ntile = (int)((vocab + kMarkovTileN - 1) / kMarkovTileN);
}

sv_status set_error(sv_status st, const char *msg)
{
    if (st == SV_OK) return ok();
    return fail(st, "%s", msg);
}

sv_status verify_args_ok(const sv_ctx *ctx, const void *p, sv_dtype pd, const void *q, sv_dtype qd,
                         const int32_t *draft, int B, int gamma, int64_t V, float T, const int32_t *accepted_len,
                         const int32_t *out_tokens, const char *fn)
{
    return check_verify_args(ctx, p, pd, q, qd, draft, B, gamma, V, T, accepted_len, out_tokens, fn);
}

VerifyArgs verify_args(const void *p, sv_dtype pd, const void *q, sv_dtype qd, const int32_t *draft,
                       const int32_t *verify_len, int B, int gamma, int64_t V, float T, uint64_t seed,
                       uint64_t offset, const float *uniforms, int32_t *accepted_len, int32_t *out_tokens,
                       const sv_diag *diag)
{
    return make_args(p, pd, q, qd, draft, verify_len, B, gamma, V, T, seed, offset, uniforms, accepted_len,
                     out_tokens, diag, false);
}

}  // namespace svh

extern "C" {

const char *spec_verify_last_error(void) { return g_err; }

sv_status spec_verify_create(sv_ctx **out, int device, int max_batch, int max_gamma, int64_t vocab,
                             int max_rank)
{
    if (!out) return fail(SV_ERR_INVALID, "spec_verify_create: out is NULL");
    *out = nullptr;
    if (max_batch <= 0) return fail(SV_ERR_INVALID, "spec_verify_create: max_batch must be > 0");
    if (max_gamma < 0 || max_gamma > svh::kMaxGamma)
        return fail(SV_ERR_INVALID, "spec_verify_create: max_gamma must be in [0, %d]", svh::kMaxGamma);
    if (vocab <= 0 || vocab >= (int64_t)1 << 31)
        return fail(SV_ERR_INVALID, "spec_verify_create: vocab must be in [1, 2^31)");
    if (max_rank != 0 && !(max_rank == 32 || max_rank == 64 || max_rank == 128 || max_rank == 256))
        return fail(SV_ERR_UNSUPPORTED, "spec_verify_create: max_rank must be 0, 32, 64, 128 or 256");
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || device < 0 || device >= ndev)
        return fail(SV_ERR_INVALID, "spec_verify_create: device %d not available", device);
    DeviceGuard guard(device);

    sv_ctx *ctx = new (std::nothrow) sv_ctx();
    if (!ctx) return fail(SV_ERR_NOMEM, "spec_verify_create: host allocation failed");
    ctx->device = device;
    ctx->max_batch = max_batch;
    ctx->max_gamma = max_gamma;
    ctx->vocab = vocab;
    ctx->max_rank = max_rank;
    int ncu = 0;
    if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || ncu <= 0)
        ncu = 256;
    ctx->num_cu = ncu;
    svh::set_geometry(ctx, vocab, (int64_t)max_batch * (2 * (int64_t)max_gamma + 1));

    const size_t rows_max = (size_t)max_batch * (2 * (size_t)max_gamma + 1);
    size_t off = 0;
    auto carve = [&](size_t bytes) {
        const size_t at = off;
        off = align_up(off + bytes, 256);
        return at;
    };
    const size_t o_part = carve(rows_max * ctx->nch1 * sizeof(float2));
    const size_t o_csum = carve((size_t)max_batch * ctx->nseg * sizeof(float));
    const size_t o_bm = carve((size_t)max_batch * (max_gamma > 0 ? max_gamma : 1) * ctx->nseg * sizeof(float));
    const size_t o_req = carve((size_t)max_batch * svh::kReqStateBytes);
    const size_t o_lp2 = carve((size_t)max_batch * (max_gamma + 1) * sizeof(float));
    const size_t o_lq2 = carve((size_t)max_batch * (max_gamma > 0 ? max_gamma : 1) * sizeof(float));
    const size_t o_wrun = carve((size_t)max_batch * (max_gamma + 1) * sizeof(double));
    const size_t o_err = carve(sizeof(uint32_t));
    const size_t o_sched = carve((size_t)max_batch * sizeof(int32_t));
    const size_t o_srank = carve((size_t)svh::kSchedMax * sizeof(int32_t));
    const size_t o_ssurv = carve((size_t)svh::kSchedMax * sizeof(double));
    const size_t o_rnnh = carve((size_t)max_batch * (max_rank > 0 ? max_rank : 1) * sizeof(uint16_t));
    const size_t o_tstate = carve(2 * (size_t)max_batch * svh::kTreeStateBytes);
    const size_t o_tseg = carve(2 * (size_t)max_batch * ctx->nseg * sizeof(float));
    size_t o_mkpart = 0, o_mkq = 0, o_mklse = 0, o_mkzx = 0;
    if (max_rank > 0) {
        o_mkpart = carve((size_t)max_batch * ctx->ntile * sizeof(float2));
        o_mkq = carve((size_t)max_batch * (size_t)vocab * sizeof(float));
        o_mklse = carve((size_t)max_batch * (max_gamma > 0 ? max_gamma : 1) * sizeof(float));
        o_mkzx = carve((size_t)max_batch * (max_gamma > 0 ? max_gamma : 1) * sizeof(float));
    }
    void *base = nullptr;
    if (hipMalloc(&base, off) != hipSuccess) {
        delete ctx;
        return fail(SV_ERR_NOMEM, "spec_verify_create: hipMalloc of %zu bytes failed", off);
    }
    if (hipMemset(base, 0, off) != hipSuccess) {
        (void)hipFree(base);
        delete ctx;
        return fail(SV_ERR_HIP, "spec_verify_create: hipMemset failed");
    }
    char *b = (char *)base;
    ctx->ws.base = base;
    ctx->ws.bytes = off;
    ctx->ws.part = (float2 *)(b + o_part);
    ctx->ws.csum = (float *)(b + o_csum);
    ctx->ws.bm = (float *)(b + o_bm);
    ctx->ws.req = (void *)(b + o_req);
    ctx->ws.lp2 = (float *)(b + o_lp2);
    ctx->ws.lq2 = (float *)(b + o_lq2);
    ctx->ws.wrun = (double *)(b + o_wrun);
    ctx->ws.errword = (uint32_t *)(b + o_err);
    ctx->ws.sched_len = (int32_t *)(b + o_sched);
    ctx->ws.sched_rank = (int32_t *)(b + o_srank);
    ctx->ws.sched_surv = (double *)(b + o_ssurv);
    ctx->ws.rnn_h = (uint16_t *)(b + o_rnnh);
    ctx->ws.tree_state = (void *)(b + o_tstate);
    ctx->ws.tree_seg = (float *)(b + o_tseg);
    ctx->ws.mk_part = max_rank > 0 ? (float2 *)(b + o_mkpart) : nullptr;
    ctx->ws.mk_q = max_rank > 0 ? (float *)(b + o_mkq) : nullptr;
    ctx->ws.mk_lse2 = max_rank > 0 ? (float *)(b + o_mklse) : nullptr;
    ctx->ws.mk_zx = max_rank > 0 ? (float *)(b + o_mkzx) : nullptr;
    *out = ctx;
    return ok();
}

namespace {

void profile_free(sv_ctx *ctx)
{
    SvProfile &p = ctx->prof;
    for (int i = 0; i < p.cap; ++i) {
        (void)hipEventDestroy(p.ev0[i]);
        (void)hipEventDestroy(p.ev1[i]);
    }
    delete[] p.ev0;
    delete[] p.ev1;
    delete[] p.kind;
    p = SvProfile();
}

}  // namespace

void spec_verify_destroy(sv_ctx *ctx)
{
    if (!ctx) return;
    {
        DeviceGuard guard(ctx->device);
        profile_free(ctx);
        if (ctx->ws.base) (void)hipFree(ctx->ws.base);
    }
    delete ctx;
}

sv_status spec_verify_profile_enable(sv_ctx *ctx, int enable)
{
    if (!ctx) return fail(SV_ERR_INVALID, "spec_verify_profile_enable: ctx is NULL");
    DeviceGuard guard(ctx->device);
    if (!enable) {
        profile_free(ctx);
        return ok();
    }
    if (ctx->prof.on) return ok();
    constexpr int kCap = 4096;
    SvProfile &p = ctx->prof;
    p.ev0 = new (std::nothrow) hipEvent_t[kCap];
    p.ev1 = new (std::nothrow) hipEvent_t[kCap];
    p.kind = new (std::nothrow) int[kCap];
    if (!p.ev0 || !p.ev1 || !p.kind) {
        profile_free(ctx);
        return fail(SV_ERR_NOMEM, "spec_verify_profile_enable: host allocation failed");
    }
    for (int i = 0; i < kCap; ++i) {
        if (hipEventCreate(&p.ev0[i]) != hipSuccess || hipEventCreate(&p.ev1[i]) != hipSuccess) {
            p.cap = i;
            profile_free(ctx);
            return fail(SV_ERR_HIP, "spec_verify_profile_enable: hipEventCreate failed");
        }
        p.cap = i + 1;
    }
    p.n = 0;
    p.on = true;
    return ok();
}

sv_status spec_verify_profile_read(sv_ctx *ctx, double *total_ms, int64_t *launches)
{
    if (!ctx || !total_ms || !launches)
        return fail(SV_ERR_INVALID, "spec_verify_profile_read: ctx, total_ms and launches are required");
    for (int k = 0; k < SV_KERNEL_COUNT; ++k) {
        total_ms[k] = 0.0;
        launches[k] = 0;
    }
    SvProfile &p = ctx->prof;
    if (!p.on) return fail(SV_ERR_INVALID, "spec_verify_profile_read: profiling is not enabled");
    DeviceGuard guard(ctx->device);
    for (int i = 0; i < p.n; ++i) {
        hipError_t e = hipEventSynchronize(p.ev1[i]);
        float ms = 0.0f;
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, p.ev0[i], p.ev1[i]);
        if (e != hipSuccess) {
            p.n = 0;
            return fail(SV_ERR_HIP, "spec_verify_profile_read: %s", hipGetErrorString(e));
        }
        total_ms[p.kind[i]] += ms;
        launches[p.kind[i]] += 1;
    }
    p.n = 0;
    return ok();
}

sv_status spec_verify_device_status(sv_ctx *ctx, hipStream_t stream, uint32_t *flags)
{
    if (!ctx || !flags) return fail(SV_ERR_INVALID, "spec_verify_device_status: ctx and flags are required");
    DeviceGuard guard(ctx->device);
    uint32_t h = 0;
    hipError_t e = hipMemcpyAsync(&h, ctx->ws.errword, sizeof(h), hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipMemsetAsync(ctx->ws.errword, 0, sizeof(uint32_t), stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return fail(SV_ERR_HIP, "spec_verify_device_status: %s", hipGetErrorString(e));
    *flags = h;
    return ok();
}

sv_status spec_verify_run(sv_ctx *ctx, hipStream_t stream, const void *p_logits, sv_dtype p_dtype,
                          const void *q_logits, sv_dtype q_dtype, const int32_t *draft_tokens,
                          const int32_t *verify_len, int B, int gamma, int64_t V, float temperature,
                          uint64_t seed, uint64_t offset, const float *uniforms, int32_t *accepted_len,
                          int32_t *out_tokens, const sv_diag *diag)
{
    sv_status st = check_verify_args(ctx, p_logits, p_dtype, q_logits, q_dtype, draft_tokens, B, gamma, V,
                                     temperature, accepted_len, out_tokens, "spec_verify_run");
    if (st != SV_OK) return st;
    DeviceGuard guard(ctx->device);
    const svh::VerifyArgs a = make_args(p_logits, p_dtype, q_logits, q_dtype, draft_tokens, verify_len, B,
                                        gamma, V, temperature, seed, offset, uniforms, accepted_len,
                                        out_tokens, diag, false);
    if ((st = check_launch(svh::launch_token_verify(ctx, a, stream), "token verification")) != SV_OK) return st;
    return ok();
}

static sv_status schedule_common(sv_ctx *ctx, hipStream_t stream, const float *conf, const svh::StsTemps &sts,
                                 int B, int gamma, float sps_a, float sps_k, int32_t *verify_len, double *expected,
                                 const char *who)
{
    if (!ctx) return fail(SV_ERR_INVALID, "%s: ctx is NULL", who);
    if (B <= 0 || B > ctx->max_batch || gamma < 0 || gamma > ctx->max_gamma)
        return fail(SV_ERR_INVALID, "%s: B=%d or gamma=%d out of range", who, B, gamma);
    if (B > svh::kSchedMax || (int64_t)B * gamma > svh::kSchedMax)
        return fail(SV_ERR_UNSUPPORTED, "%s: B and B*gamma must be <= %d", who, svh::kSchedMax);
    if (!verify_len || (gamma > 0 && !conf))
        return fail(SV_ERR_INVALID, "%s: conf and verify_len are required", who);
    if (!(sps_a > 0.0f) || !(sps_k > 0.0f) || !std::isfinite(sps_a) || !std::isfinite(sps_k))
        return fail(SV_ERR_INVALID, "%s: sps_a and sps_k must be finite and > 0", who);
    DeviceGuard guard(ctx->device);
    sv_status st = check_launch(svh::launch_schedule(ctx, conf, sts, B, gamma, sps_a, sps_k, verify_len, expected,
                                                     stream),
                                "scheduler");
    return st != SV_OK ? st : ok();
}

sv_status spec_schedule_run(sv_ctx *ctx, hipStream_t stream, const float *conf, int B, int gamma,
                            float sps_a, float sps_k, int32_t *verify_len, double *expected)
{
    svh::StsTemps sts{};
    return schedule_common(ctx, stream, conf, sts, B, gamma, sps_a, sps_k, verify_len, expected,
                           "spec_schedule_run");
}

sv_status spec_schedule_sts_run(sv_ctx *ctx, hipStream_t stream, const float *conf_logits,
                                const float *temperatures, int B, int gamma, float sps_a, float sps_k,
                                int32_t *verify_len, double *expected)
{
    svh::StsTemps sts{};
    sts.on = 1;
    if (!ctx) return fail(SV_ERR_INVALID, "spec_schedule_sts_run: ctx is NULL");
    if (gamma < 0 || gamma > ctx->max_gamma)
        return fail(SV_ERR_INVALID, "spec_schedule_sts_run: gamma=%d out of range", gamma);
    if (gamma > 0 && !temperatures)
        return fail(SV_ERR_INVALID, "spec_schedule_sts_run: temperatures are required");
    for (int i = 0; i < gamma; ++i) {
        if (!(temperatures[i] > 0.0f) || !std::isfinite(temperatures[i]))
            return fail(SV_ERR_INVALID, "spec_schedule_sts_run: temperature %d (%g) must be finite and > 0", i,
                        (double)temperatures[i]);
        sts.t[i] = temperatures[i];
    }
    return schedule_common(ctx, stream, conf_logits, sts, B, gamma, sps_a, sps_k, verify_len, expected,
                           "spec_schedule_sts_run");
}

sv_status spec_blockverify_run(sv_ctx *ctx, hipStream_t stream, const void *p_logits, sv_dtype p_dtype,
                               const void *q_logits, sv_dtype q_dtype, const int32_t *draft_tokens,
                               const int32_t *verify_len, const float *conf, float sps_a, float sps_k,
                               int32_t *verify_len_out, int B, int gamma, int64_t V, float temperature,
                               uint64_t seed, uint64_t offset, const float *uniforms, int32_t *accepted_len,
                               int32_t *out_tokens, const sv_diag *diag)
{
    sv_status st = check_verify_args(ctx, p_logits, p_dtype, q_logits, q_dtype, draft_tokens, B, gamma, V,
                                     temperature, accepted_len, out_tokens, "spec_blockverify_run");
    if (st != SV_OK) return st;
    DeviceGuard guard(ctx->device);
    const int32_t *vl = verify_len;
    if (conf) {
        int32_t *dst = verify_len_out ? verify_len_out : ctx->ws.sched_len;
        st = spec_schedule_run(ctx, stream, conf, B, gamma, sps_a, sps_k, dst, nullptr);
        if (st != SV_OK) return st;
        vl = dst;
    }
    const svh::VerifyArgs a = make_args(p_logits, p_dtype, q_logits, q_dtype, draft_tokens, vl, B, gamma, V,
                                        temperature, seed, offset, uniforms, accepted_len, out_tokens, diag,
                                        true);
    if ((st = run_verify(ctx, a, stream, svh::launch_block_tail, "block thresholds / residual sampler")) != SV_OK)
        return st;
    return ok();
}

sv_status markov_draft_run(sv_ctx *ctx, hipStream_t stream, const void *base_logits, const void *U,
                           const void *W, int R, const int32_t *x0, int B, int gamma, int64_t V,
                           float temperature, uint64_t seed, uint64_t offset, const float *uniforms,
                           int32_t *draft_tokens, float *q_logits, float *lse_q)
{
    sv_status st = check_markov_args(ctx, base_logits, U, W, R, x0, B, gamma, V, temperature, draft_tokens,
                                     "markov_draft_run");
    if (st != SV_OK) return st;
    if (q_logits && !aligned(q_logits, 4))
        return fail(SV_ERR_INVALID, "markov_draft_run: q_logits must be 4-byte aligned");
    DeviceGuard guard(ctx->device);
    svh::MarkovArgs a = make_markov_args(base_logits, U, W, R, x0, B, gamma, V, temperature, seed, offset,
                                         uniforms, draft_tokens, q_logits, lse_q);
    st = check_launch(svh::launch_markov(ctx, a, stream), "Markov sampler");
    return st != SV_OK ? st : ok();
}

sv_status tree_verify_run(sv_ctx *ctx, hipStream_t stream, const void *p_logits, sv_dtype p_dtype,
                          const void *q_logits, sv_dtype q_dtype, const int32_t *tokens, const int32_t *parents,
                          int N, int B, int64_t V, float temperature, uint64_t seed, uint64_t offset,
                          const float *uniforms, int32_t *accepted_len, int32_t *out_tokens,
                          int32_t *accepted_nodes, const sv_diag *diag)
{
    const char *fn = "tree_verify_run";
    if (!ctx) return fail(SV_ERR_INVALID, "%s: ctx is NULL", fn);
    if (N < 0 || N > ctx->max_gamma)
        return fail(SV_ERR_INVALID, "%s: N=%d nodes out of range [0, max_gamma=%d]", fn, N, ctx->max_gamma);
    if (N > 0 && !parents) return fail(SV_ERR_INVALID, "%s: parents are required", fn);
    // topology: parents come first; children in index order; q rows of the
    // nodes with children in node order
    svh::TreeTopo t;
    std::memset(&t, 0, sizeof t);
    t.N = N;
    int depth[svh::kMaxGamma + 1];
    depth[0] = 0;
    int8_t last[svh::kMaxGamma + 1];
    for (int n = 0; n <= N; ++n) {
        t.first_child[n] = -1;
        t.next_sib[n] = -1;
        t.qrow[n] = -1;
        last[n] = -1;
    }
    t.parent[0] = -1;
    for (int m = 1; m <= N; ++m) {
        const int32_t par = parents[m - 1];
        if (par < 0 || par >= m)
            return fail(SV_ERR_INVALID, "%s: parents[%d]=%d must lie in [0, %d]", fn, m - 1, par, m - 1);
        t.parent[m] = (int8_t)par;
        depth[m] = depth[par] + 1;
        t.D = depth[m] > t.D ? depth[m] : t.D;
        if (last[par] < 0) t.first_child[par] = (int8_t)m;
        else t.next_sib[last[par]] = (int8_t)m;
        last[par] = (int8_t)m;
    }
    for (int n = 0; n <= N; ++n)
        if (t.first_child[n] >= 0) t.qrow[n] = (int8_t)t.NQ++;
    // passes a walk can need: at each node on the path c - 1 rejections that
    // leave a sibling to try (c its children), then the draw and one retry of
    // the draw from p; one more round consumes the last sums
    {
        int nch[svh::kMaxGamma + 1] = {0};
        for (int m = 1; m <= N; ++m) nch[t.parent[m]] += 1;
        int above[svh::kMaxGamma + 1];
        above[0] = 0;
        int most = 0;
        for (int v = 0; v <= N; ++v) {
            if (v > 0) above[v] = above[t.parent[v]] + nch[t.parent[v]] - 1;
            const int here = above[v] + (nch[v] > 0 ? nch[v] - 1 : 0);
            most = here > most ? here : most;
        }
        t.rounds = most + 2 + 1;
    }
    // the row checks of a draft call with gamma = N (q has NQ <= N rows)
    sv_status st = check_verify_args(ctx, p_logits, p_dtype, q_logits, q_dtype, tokens, B, N, V, temperature,
                                     accepted_len, out_tokens, fn);
    if (st != SV_OK) return st;
    if (ctx->nseg > svh::kTailMaxSeg)
        return fail(SV_ERR_UNSUPPORTED, "%s: V=%lld exceeds the tree walk's segment table", fn, (long long)V);
    DeviceGuard guard(ctx->device);
    svh::VerifyArgs a = make_args(p_logits, p_dtype, q_logits, q_dtype, tokens, nullptr, B, N, V, temperature,
                                  seed, offset, uniforms, accepted_len, out_tokens, diag, false);
    a.np_rows = N + 1;
    a.nq_rows = t.NQ;
    if ((st = check_launch(svh::launch_rowstats(ctx, a, stream), "row statistics")) != SV_OK) return st;
    if ((st = check_launch(svh::launch_tree_tail(ctx, a, t, accepted_nodes, stream), "tree walk")) != SV_OK)
        return st;
    return ok();
}

sv_status rnn_draft_run(sv_ctx *ctx, hipStream_t stream, const void *base_logits, const void *U, const void *W,
                        const void *A, int R, const int32_t *x0, int B, int gamma, int64_t V, float temperature,
                        uint64_t seed, uint64_t offset, const float *uniforms, int32_t *draft_tokens,
                        float *q_logits, float *lse_q, uint16_t *states)
{
    sv_status st = check_markov_args(ctx, base_logits, U, W, R, x0, B, gamma, V, temperature, draft_tokens,
                                     "rnn_draft_run");
    if (st != SV_OK) return st;
    if (!A) return fail(SV_ERR_INVALID, "rnn_draft_run: A is required");
    if (!aligned(A, 16) || (states && !aligned(states, 2)))
        return fail(SV_ERR_INVALID, "rnn_draft_run: A must be 16-byte aligned and states 2-byte aligned");
    if (q_logits && !aligned(q_logits, 4))
        return fail(SV_ERR_INVALID, "rnn_draft_run: q_logits must be 4-byte aligned");
    DeviceGuard guard(ctx->device);
    svh::MarkovArgs a = make_markov_args(base_logits, U, W, R, x0, B, gamma, V, temperature, seed, offset,
                                         uniforms, draft_tokens, q_logits, lse_q);
    a.A = (const uint16_t *)A;
    a.hstate = ctx->ws.rnn_h;
    a.states_out = states;
    a.fused = q_logits == nullptr;   // no z rows wanted: the draw rebuilds its tile
    st = check_launch(svh::launch_markov(ctx, a, stream), "RNN-head sampler");
    return st != SV_OK ? st : ok();
}

sv_status markov_verify_run(sv_ctx *ctx, hipStream_t stream, const void *base_logits, const void *U,
                            const void *W, int R, const int32_t *x0, const void *p_logits, sv_dtype p_dtype,
                            int B, int gamma, int64_t V, float temperature, uint64_t draft_seed,
                            uint64_t verify_seed, uint64_t offset, int32_t *draft_tokens, int32_t *accepted_len,
                            int32_t *out_tokens, float *lse_q, const sv_diag *diag)
{
    sv_status st = check_markov_args(ctx, base_logits, U, W, R, x0, B, gamma, V, temperature, draft_tokens,
                                     "markov_verify_run");
    if (st != SV_OK) return st;
    if (!p_logits || !accepted_len || !out_tokens)
        return fail(SV_ERR_INVALID, "markov_verify_run: p_logits, accepted_len and out_tokens are required");
    if (esize_of(p_dtype) == 0) return fail(SV_ERR_UNSUPPORTED, "markov_verify_run: p dtype must be SV_BF16 or SV_F32");
    if (!aligned(p_logits, esize_of(p_dtype)))
        return fail(SV_ERR_INVALID, "markov_verify_run: p_logits must be aligned to its element size");
    DeviceGuard guard(ctx->device);
    RideGeometry ride_geometry(ctx);
    svh::VerifyArgs a = make_args(p_logits, p_dtype, nullptr, SV_F32, draft_tokens, nullptr, B, gamma, V,
                                  temperature, verify_seed, offset, nullptr, accepted_len, out_tokens, diag, false);
    a.q_esize = 4;
    a.q_lse2 = ctx->ws.mk_lse2;
    a.q_zx = ctx->ws.mk_zx;
    // 1. the draft: no z rows stored; the sampler records each row's
    //    log2-sum-exp2 and the drafted tokens' logits.  The chunk
    //    statistics of the p rows (they do not depend on the draft) ride in
    //    the draws' launches, whose few dependent round trips leave the
    //    memory system idle.
    svh::MarkovArgs m = make_markov_args(base_logits, U, W, R, x0, B, gamma, V, temperature, draft_seed, offset,
                                         nullptr, draft_tokens, nullptr, lse_q);
    m.fused = true;
    m.lse2_out = ctx->ws.mk_lse2;
    m.zx_out = ctx->ws.mk_zx;
    m.ride = svh::RowRide{a.p, a.p_esize, ctx->nch1, ctx->chunk1, a.c, ctx->ws.part,
                          (int64_t)B * (gamma + 1) * ctx->nch1};
    if ((st = check_launch(svh::launch_markov(ctx, m, stream), "Markov sampler")) != SV_OK) return st;
    // 2. verification of that draft: the scan with the sampler's q
    //    statistics, the correction / bonus weights of the rebuilt correction
    //    rows summed per tile, the draw
    if ((st = check_launch(svh::launch_markov_verify_tail(ctx, a, m, stream), "fused verification")) != SV_OK)
        return st;
    return ok();
}

}  // extern "C"
