// sv_internal.h -- host-side internals of libspecverify: the context, its
// device workspace and the kernel launchers each .hip file provides.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "spec_verify.h"

namespace svh {

// Row-statistics pass: a row of V logits is split into `nch1` chunks of
// `chunk1` elements (a multiple of 8, so chunk starts keep 16-byte alignment).
// The defaults come from a sweep on MI355X; the macros exist for re-tuning.
#ifndef SV_ROWSTATS_THREADS
#define SV_ROWSTATS_THREADS 256
#endif
#ifndef SV_ROWSTATS_CHUNK
#define SV_ROWSTATS_CHUNK 16384
#endif
#ifndef SV_ROWSTATS_NB
#define SV_ROWSTATS_NB 8
#endif
#ifndef SV_ROWSTATS_NT_LOADS
#define SV_ROWSTATS_NT_LOADS 1   // stream the logits with nontemporal loads
#endif

constexpr int kRowstatsThreads = SV_ROWSTATS_THREADS;
constexpr int kTargetChunk1 = SV_ROWSTATS_CHUNK;
constexpr int kRowstatsNB = SV_ROWSTATS_NB;   // 16-byte loads in flight per thread
#ifndef SV_ROWSTATS_COMPACT_WGS
#define SV_ROWSTATS_COMPACT_WGS 4
#endif
#ifndef SV_ROWSTATS_COMPACT_NB
#define SV_ROWSTATS_COMPACT_NB 4
#endif
constexpr int kRowstatsCompactWGsPerCU = SV_ROWSTATS_COMPACT_WGS;   // grid of the compacted variant, per CU
constexpr int kRowstatsCompactNB = SV_ROWSTATS_COMPACT_NB;          // its 16-byte loads in flight per thread
constexpr int kRowstatsCompactMaxReq = 8192;  // requests per call it lays out in LDS (64 KB)
// Correction / bonus weights and block pass 2: each wavefront sums one
// segment of kSegR elements; a workgroup covers kSegPerWG segments.
constexpr int kResidThreads = 256;
constexpr int kSegR = 2048;
constexpr int kSegPerWG = kResidThreads / 64;
// Fused tails: per-request segment sums of the correction / bonus weights in
// LDS, V <= kTailMaxSeg * kSegR tokens.
constexpr int kTailMaxSeg = 4096;
// Scheduler: one workgroup sorts up to kSchedMax candidates in LDS.
constexpr int kSchedThreads = 1024;
constexpr int kSchedMax = 8192;
// Markov head: output tiles of kMarkovTileN vocabulary columns.
constexpr int kMarkovTileN = 64;
constexpr int kMarkovMaxTiles = 256 * 16;  // the draw keeps 16 tile pairs per thread: V <= 262,144
constexpr int kMaxGamma = 64;
// Scratch of the allocation-free token verification (a file-scope device
// array, one per GPU): row-chunk statistics, request state and segment sums.
#ifndef SV_NOALLOC_SCRATCH_BYTES
#define SV_NOALLOC_SCRATCH_BYTES (8u << 20)
#endif


struct Workspace {
    float2 *part;        // [rows_max * nch1] (m, s) per row chunk
    float *csum;         // [max_batch * nseg] correction/bonus segment sums
    float *bm;           // [max_batch * max_gamma * nseg] block residual-mass partials
    void *req;           // [max_batch] per-request state (ReqG, verify.hip)
    float *lp2;          // [max_batch * (max_gamma + 1)] log2-sum-exp2 of verified p rows
    float *lq2;          // [max_batch * max_gamma]       ... and q rows
    double *wrun;        // [max_batch * (max_gamma + 1)] block running ratios w_0..w_L
    uint32_t *errword;   // [1] OR of SV_FLAG_* bits
    int32_t *sched_len;  // [max_batch] scheduler output when the caller gives none
    int32_t *sched_rank; // [kSchedMax] candidate ranks, zero between calls
    double *sched_surv;  // [kSchedMax] candidate survival products
    uint16_t *rnn_h;     // [max_batch, max_rank] bf16 RNN-head state
    float2 *mk_part;     // [max_batch * ntile] Markov tile (m, s) partials; after the
                         // fused path's draft, its correction / bonus tile sums (floats)
    float *mk_q;         // [max_batch * V] Markov logits of the current position when
                         // the caller does not keep them
    float *mk_lse2;      // [max_batch * max_gamma] fused path: draft row log2-sum-exp2
    float *mk_zx;        // [max_batch * max_gamma] fused path: drafted tokens' logits
    void *tree_state;    // [2][max_batch] kTreeStateBytes: tree walk state by round parity
    float *tree_seg;     // [2][max_batch * nseg] tree walk segment sums by round parity
    void *base;          // single allocation backing all of the above
    size_t bytes;
};

}  // namespace svh

// Optional per-kernel event timing (spec_verify_profile_*).
struct SvProfile {
    bool on = false;
    int cap = 0;             // event pairs in the pool
    int n = 0;               // pairs recorded since the last read
    hipEvent_t *ev0 = nullptr, *ev1 = nullptr;
    int *kind = nullptr;
};

struct sv_ctx {
    int device;
    int max_batch;
    int max_gamma;
    int64_t vocab;
    int max_rank;
    int num_cu;          // compute units of the device
    int nch1;            // row-statistics chunks per row
    int64_t chunk1;      // elements per row-statistics chunk
    int nseg;            // residual segments (kSegR elements) per row
    int ntile;           // Markov vocabulary tiles
    svh::Workspace ws;
    SvProfile prof;
};

namespace svh {

// Records the start event of a timed launch; returns the pool slot or -1.
inline int prof_begin(sv_ctx *ctx, hipStream_t s, int kind)
{
    SvProfile &p = ctx->prof;
    if (!p.on || p.n >= p.cap) return -1;
    const int slot = p.n++;
    p.kind[slot] = kind;
    (void)hipEventRecord(p.ev0[slot], s);
    return slot;
}

inline void prof_end(sv_ctx *ctx, hipStream_t s, int slot)
{
    if (slot >= 0) (void)hipEventRecord(ctx->prof.ev1[slot], s);
}

// Arguments shared by the verification launchers.
struct VerifyArgs {
    const void *p;
    const void *q;
    int p_esize;          // 2 (bf16) or 4 (fp32)
    int q_esize;
    const int32_t *draft;
    const int32_t *verify_len;   // may be null
    int B, gamma;
    int b0, nb;           // requests [b0, b0 + nb) of the batch handled by a launch
    int64_t V;
    float c;              // log2(e) / T
    uint64_t seed, offset;
    const float *uniforms;       // may be null
    int32_t *accepted_len;
    int32_t *out_tokens;
    sv_diag diag;         // device pointers, each may be null
    bool block;           // block verification
    // Draft rows that were never materialised (the fused Markov path): the
    // sampler's per-row log2-sum-exp2 of z * c and the drafted tokens' raw
    // logits replace the q row statistics.  Null otherwise.
    const float *q_lse2;  // [B, gamma]
    const float *q_zx;    // [B, gamma]
    // Row counts per request when they are not gamma + 1 and gamma (tree
    // verification: N + 1 node rows of p, one q row per node with children);
    // 0 for a draft.
    int np_rows, nq_rows;
};

// Per-request result of the acceptance scan, read by the kernels that follow.
struct ReqG {
    uint32_t flags;
    int32_t L;
    int32_t tau;
    int32_t mode;      // 0: residual weights max(wmul * p - q, 0), 1: bonus weights p
    float wmul;        // multiplier of p in the residual weights (w_tau; 1 for the token rule)
    float lp2, lq2;    // log2-sum-exp2 of p row tau+1 and q row tau+1
    float u2;          // correction / bonus uniform
};

// Row-chunk and segment geometry of a context for vocabulary `vocab` and at
// most `rows_max` verified rows per call (nch1, chunk1, nseg, ntile).
void set_geometry(sv_ctx *ctx, int64_t vocab, int64_t rows_max);
// Row-statistics chunks of about `target` elements (a multiple of 8) over a
// row of `vocab`: their count and length.
void chunk_geometry(int64_t vocab, int64_t target, int *nch1, int64_t *chunk1);
// Argument checks and argument block of token verification (api.cpp), for
// entry points defined in other files; set_error records a status and
// message for spec_verify_last_error (SV_OK clears it).
sv_status set_error(sv_status st, const char *msg);
sv_status verify_args_ok(const sv_ctx *ctx, const void *p, sv_dtype pd, const void *q, sv_dtype qd,
                         const int32_t *draft, int B, int gamma, int64_t V, float T, const int32_t *accepted_len,
                         const int32_t *out_tokens, const char *fn);
VerifyArgs verify_args(const void *p, sv_dtype pd, const void *q, sv_dtype qd, const int32_t *draft,
                       const int32_t *verify_len, int B, int gamma, int64_t V, float T, uint64_t seed,
                       uint64_t offset, const float *uniforms, int32_t *accepted_len, int32_t *out_tokens,
                       const sv_diag *diag);

hipError_t launch_rowstats(sv_ctx *ctx, const VerifyArgs &a, hipStream_t s);
// Token verification after the row statistics: accept -> chunk sums -> select.
hipError_t launch_token_tail(sv_ctx *ctx, const VerifyArgs &a, hipStream_t s);
// The whole token verification: row statistics then the tail, or, for a
// small problem (one chunk per row, few rows), one launch doing both.
hipError_t launch_token_verify(sv_ctx *ctx, const VerifyArgs &a, hipStream_t s);
// Block verification after the row statistics: ratios -> residual masses ->
// thresholds -> chunk sums -> select.
hipError_t launch_block_tail(sv_ctx *ctx, const VerifyArgs &a, hipStream_t s);
// Tree topology (node 0 the root, nodes 1..N in an order where parents come
// first), shared by every request of a call.
struct TreeTopo {
    int N, NQ, D;                       // nodes, nodes with children, depth
    int8_t parent[kMaxGamma + 1];       // parent of node m >= 1
    int8_t first_child[kMaxGamma + 1];  // -1 for a leaf
    int8_t next_sib[kMaxGamma + 1];     // next child of the same parent, -1 for the last
    int8_t qrow[kMaxGamma + 1];         // q row of a node with children, else -1
    int rounds;                         // walk rounds covering the longest sequence of passes
};
// Bytes of one request's walk state in the tree workspace.
constexpr size_t kTreeStateBytes = 3072;
// Tree verification after the row statistics (a.np_rows = N + 1, a.nq_rows =
// NQ): one workgroup per request walks the tree and draws the final token.
hipError_t launch_tree_tail(sv_ctx *ctx, const VerifyArgs &a, const TreeTopo &t, int32_t *nodes_out,
                            hipStream_t s);
constexpr size_t kReqStateBytes = 32;
static_assert(sizeof(ReqG) == kReqStateBytes, "request state layout");
// Per-position temperatures of sequential temperature scaling, passed by
// value; with on == 0 the scheduler reads confidences, otherwise log-odds.
struct StsTemps {
    float t[kMaxGamma];
    int on;
};
hipError_t launch_schedule(sv_ctx *ctx, const float *conf, const StsTemps &sts, int B, int gamma, float sps_a,
                           float sps_k, int32_t *verify_len, double *expected, hipStream_t s);

// Chunk statistics of the target rows carried by the draws of the fused
// Markov draft -> verification path: item i is chunk i % nch1 of p row
// i / nch1 ([B, gamma + 1] rows), written to part[i] as the row-statistics
// pass would.  items == 0: nothing rides.
struct RowRide {
    const void *p;
    int pes;               // 2 (bf16) or 4 (fp32)
    int nch1;
    int64_t chunk1;
    float c;
    float2 *part;
    int64_t items;
};

struct MarkovArgs {
    const uint16_t *base;  // [B, gamma, V] bf16
    const uint16_t *U;     // [V, R]
    const uint16_t *W;     // [V, R]: the transition matrix stored vocabulary-major
    int R;
    const int32_t *x0;
    int B, gamma;
    int64_t V;
    float c;               // log2(e) / T
    uint64_t seed, offset;
    const float *uniforms;
    int32_t *draft;
    float *q_logits;       // may be null
    float *lse_q;          // may be null
    // Fused draft -> verification: no z row is stored; the draw rebuilds the
    // 64 logits of its chosen tile with the same MFMA sequence, and records
    // per (request, position) the row's log2-sum-exp2 of z * c and the drawn
    // token's raw logit.
    bool fused;
    float *lse2_out;       // [B, gamma] (fused)
    float *zx_out;         // [B, gamma] (fused)
    // RNN head (A != null): the contraction's left operand is the bf16 state
    // hb_k instead of U[x_{k-1}]; hb_1 = bf16(tanh(U[x_0])) is formed where it
    // is read, later states come from hstate, written by the draw of the
    // previous position.
    const uint16_t *A;     // [R, R] bf16, linear-layer layout: A[j][r] takes state entry r into j
    uint16_t *hstate;      // [B, R] bf16 workspace
    uint16_t *states_out;  // [B, gamma, R] bf16 or null
    RowRide ride;          // target-row statistics spread over the gamma draws
};

hipError_t launch_markov(sv_ctx *ctx, const MarkovArgs &a, hipStream_t s);
// Fused verification's correction / bonus draw after the acceptance scan
// (req): the contraction's residual mode sums every request's correction /
// bonus weights per vocabulary tile, then one workgroup per request draws
// the token from those sums and writes its outputs.
hipError_t launch_markov_resid(sv_ctx *ctx, const MarkovArgs &a, const VerifyArgs &v, const ReqG *req,
                               hipStream_t s);
// Fused Markov draft -> verification after the p row statistics: the
// acceptance scan (token rule, q statistics from the sampler), the correction
// rows rebuilt, then the correction / bonus draw.
hipError_t launch_markov_verify_tail(sv_ctx *ctx, const VerifyArgs &a, const MarkovArgs &m, hipStream_t s);

}  // namespace svh
