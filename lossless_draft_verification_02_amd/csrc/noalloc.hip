// noalloc.hip -- token-level verification without a context and without any
// allocation, for callers that cannot allocate device memory (code under HIP
// graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The kernels are spec_verify_run's; their per-call scratch (row-chunk
// statistics, per-request state, correction-weight segment sums, the device
// error word) lives in one file-scope device array instead of a context
// workspace.  Host code never passes the array's name to a kernel: the name
// is a host-side stand-in, so the device address is looked up once per device
// with hipGetSymbolAddress (with that device current) and kept.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <mutex>

#include "spec_verify.h"
#include "sv_internal.h"

namespace {

constexpr size_t kScratchBytes = SV_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

// One copy per GPU the library runs on, held until the process ends.
__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_lock;
void *g_scratch[kMaxDevices];   // device address of `scratch` on each device, once looked up

// Device address of the current device's scratch array (looked up on the
// first call on that device); nullptr and a message on failure.
void *scratch_on(int dev, char *msg, size_t len)
{
    if (dev < 0 || dev >= kMaxDevices) {
        std::snprintf(msg, len, "spec_verify_run_noalloc: device %d beyond the library's %d-device table", dev,
                      kMaxDevices);
        return nullptr;
    }
    std::lock_guard<std::mutex> g(g_lock);
    if (!g_scratch[dev]) {
        void *ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr) {
            std::snprintf(msg, len, "spec_verify_run_noalloc: hipGetSymbolAddress: %s", hipGetErrorString(e));
            return nullptr;
        }
        g_scratch[dev] = ptr;
    }
    return g_scratch[dev];
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace

extern "C" sv_status spec_verify_run_noalloc(hipStream_t stream, const void *p_logits, sv_dtype p_dtype,
                                             const void *q_logits, sv_dtype q_dtype,
                                             const int32_t *draft_tokens, const int32_t *verify_len, int B,
                                             int gamma, int64_t V, float temperature, uint64_t seed,
                                             uint64_t offset, const float *uniforms, int32_t *accepted_len,
                                             int32_t *out_tokens, const sv_diag *diag)
{
    const char *fn = "spec_verify_run_noalloc";
    char msg[256];
    if (gamma < 0 || gamma > svh::kMaxGamma) {
        std::snprintf(msg, sizeof msg, "%s: gamma=%d outside [0, %d]", fn, gamma, svh::kMaxGamma);
        return svh::set_error(SV_ERR_INVALID, msg);
    }
    if (V <= 0 || V >= ((int64_t)1 << 31)) {
        std::snprintf(msg, sizeof msg, "%s: V=%lld outside [1, 2^31)", fn, (long long)V);
        return svh::set_error(SV_ERR_INVALID, msg);
    }
    if (B <= 0) {
        std::snprintf(msg, sizeof msg, "%s: B=%d must be > 0", fn, B);
        return svh::set_error(SV_ERR_INVALID, msg);
    }
    // a context on the stack describing this call, its workspace carved from
    // the scratch array
    sv_ctx ctx;
    ctx.max_batch = B;
    ctx.max_gamma = gamma;
    ctx.vocab = V;
    ctx.max_rank = 0;
    sv_status st = svh::verify_args_ok(&ctx, p_logits, p_dtype, q_logits, q_dtype, draft_tokens, B, gamma, V,
                                       temperature, accepted_len, out_tokens, fn);
    if (st != SV_OK) return st;   // the message is recorded
    const int64_t rows = (int64_t)B * (2 * (int64_t)gamma + 1);
    svh::set_geometry(&ctx, V, rows);
    const size_t o_part = 0;
    const size_t o_csum = align_up(o_part + (size_t)rows * ctx.nch1 * sizeof(float2), 256);
    const size_t o_req = align_up(o_csum + (size_t)B * ctx.nseg * sizeof(float), 256);
    const size_t o_err = align_up(o_req + (size_t)B * svh::kReqStateBytes, 256);
    const size_t need = align_up(o_err + sizeof(uint32_t), 256);
    if (need > kScratchBytes) {
        std::snprintf(msg, sizeof msg,
                      "%s: B=%d, gamma=%d, V=%lld needs %zu bytes of scratch, above its %zu-byte maximum; "
                      "use spec_verify_run with a context",
                      fn, B, gamma, (long long)V, need, kScratchBytes);
        return svh::set_error(SV_ERR_UNSUPPORTED, msg);
    }
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        std::snprintf(msg, sizeof msg, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
        return svh::set_error(SV_ERR_HIP, msg);
    }
    char *base = (char *)scratch_on(dev, msg, sizeof msg);
    if (!base) return svh::set_error(SV_ERR_HIP, msg);
    int ncu = 0;
    if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu <= 0) ncu = 256;
    ctx.device = dev;
    ctx.num_cu = ncu;
    ctx.ws = svh::Workspace{};
    ctx.ws.part = (float2 *)(base + o_part);
    ctx.ws.csum = (float *)(base + o_csum);
    ctx.ws.req = (void *)(base + o_req);
    ctx.ws.errword = (uint32_t *)(base + o_err);
    ctx.ws.base = base;
    ctx.ws.bytes = need;
    // token verification reads none of the block, scheduler, Markov or tree
    // buffers (they stay null)
    const svh::VerifyArgs a = svh::verify_args(p_logits, p_dtype, q_logits, q_dtype, draft_tokens, verify_len, B,
                                               gamma, V, temperature, seed, offset, uniforms, accepted_len,
                                               out_tokens, diag);
    e = svh::launch_token_verify(&ctx, a, stream);
    if (e != hipSuccess) {
        std::snprintf(msg, sizeof msg, "%s: launch failed: %s", fn, hipGetErrorString(e));
        return svh::set_error(SV_ERR_HIP, msg);
    }
    return svh::set_error(SV_OK, "");
}
