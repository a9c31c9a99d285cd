// Internal interface between the C-ABI host layer (lce_api.cpp) and the
// kernel translation units.  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lce {

// Arguments of one cross-entropy call, after validation.
struct CEArgs {
    void *logits;            // [n, ld] in place
    int64_t ld;              // elements
    int64_t n;
    int64_t V;
    const int64_t *labels;
    // labels whose valid count is the mean's denominator (the rows' own labels
    // for a plain call; every token's labels for a chunk of a fused-linear call)
    const int64_t *count_labels;
    int64_t count_n;
    int64_t ignore_index;
    float eps;               // label smoothing
    float softcap;           // 0 = off
    int reduction;           // lce_reduction
    const float *grad_out;   // NULL = 1.0
    float *loss_tok;         // [n]
    float *loss_out;         // scalar or NULL
    int64_t *argmax_out;     // [n] or NULL
    int64_t *counts;         // [3]
    void *workspace;         // tagged counters + per-workgroup partials (any prior contents)
};

// Threads per row workgroup of the register-resident path.
constexpr int kRowThreads = 1024;
// Rounds (1024 x 16-byte vectors) of a row the resident path holds: up to 16
// in VGPRs (64 per lane) plus up to 9 in LDS (144 KB of the 160 KB per CU).
constexpr int kMaxRegRounds = 16;
constexpr int kMaxLdsRounds = 9;
// Upper bound on persistent workgroups (sizes the workspace partials).
constexpr int kMaxRowGroups = 4096;
// Upper bound on the half-row kernel's workgroups (two per row in flight).
constexpr int kHalfMaxGroups = 512;
// Workspace: 256-byte header (tagged counters) + 16 bytes per workgroup, then,
// 256-byte aligned, two 64-byte exchange records per half-row workgroup.
constexpr size_t ce_records_offset(int64_t n) {
    return (256 + 16 * static_cast<size_t>(n < kMaxRowGroups ? (n > 0 ? n : 1) : kMaxRowGroups) + 255) &
           ~static_cast<size_t>(255);
}
constexpr size_t ce_workspace_bytes(int64_t n) {
    return ce_records_offset(n) + 128 * static_cast<size_t>(n < kHalfMaxGroups / 2 ? 2 * (n > 0 ? n : 1)
                                                                                      : kHalfMaxGroups);
}

// Enqueue count + row kernels.  is_bf16 selects the element type.
hipError_t launch_ce_fwd_bwd(const CEArgs &a, bool is_bf16, hipStream_t stream);

// Enqueue the read-only argmax sweep (counts zeroed/filled too).
hipError_t launch_ce_argmax(const void *logits, int64_t ld, bool is_bf16, const int64_t *labels,
                            int64_t n, int64_t V, int64_t ignore_index, int64_t *argmax_out,
                            int64_t *counts, hipStream_t stream);

// Whether a shape takes the half-row kernel, and its rounds of 960 vectors per half.
bool ce_half_plan(const void *logits, int64_t ld, bool is_bf16, int64_t n, int64_t V, int *kh);

// Which row kernel a shape takes: rounds in VGPRs (*kr) and LDS (*kl), whether
// its rows are read through aligned windows (*ua), or false for the generic
// streaming kernel.
bool ce_resident_plan(const void *logits, int64_t ld, bool is_bf16, int64_t V, int *kr, int *kl, bool *ua);

// counts = {n_valid, 0, n_bad} over labels[0, n); clears the three counter words at
// ticket and *loss_out when given.
hipError_t launch_ce_count(const int64_t *labels, int64_t n, int64_t V, int64_t ignore_index, int64_t *counts,
                           unsigned long long *ticket, float *loss_out, hipStream_t stream);

// loss_out = mean (over counts[0]) or sum of loss_tok[0, n), 0 for 'none'; one
// workgroup, fixed-order fp64 sum.
hipError_t launch_loss_fold(const float *loss_tok, int64_t n, const int64_t *counts, int reduction, float *loss_out,
                            hipStream_t stream);

// ---- split cross-entropy: shard statistics, combine, gradient ----------------

// One stats record per row and shard: 8 floats (max z, sums of e^{z-max} and of
// e^{z-max} z without the target, sum z, argmax value, global argmax index as
// int bits, target z, target-present flag).
constexpr int kStatsFloats = 8;
hipError_t launch_ce_stats(const void *logits, int64_t ld, bool is_bf16, const int64_t *labels, int64_t n,
                           int64_t Vs, int64_t v0, int64_t ignore_index, float softcap, float *stats,
                           hipStream_t stream);
// Record of row i, shard k at stats + (k * shard_stride + i * row_stride) * 8.
hipError_t launch_ce_combine(const float *stats, int64_t shards, int64_t shard_stride, int64_t row_stride,
                             const int64_t *labels, int64_t n, int64_t V,
                             int64_t ignore_index, float eps, int reduction, float *lse, float *q, float *loss_tok,
                             float *loss_out, float *logp, float *ent, int64_t *argmax_out, int64_t *counts,
                             hipStream_t stream);
hipError_t launch_ce_grad(void *logits, int64_t ld, bool is_bf16, const int64_t *labels, int64_t n, int64_t Vs,
                          int64_t v0, int64_t V, int64_t ignore_index, float eps, float softcap, int reduction,
                          const float *grad_out, const float *lse, const float *q, const int64_t *counts,
                          hipStream_t stream);

// ---- fused linear cross-entropy ----------------------------------------------

// Compute units of the current device (cached per device).
int device_cu_count();

// Most K splits of the grad_hidden GEMM (K = V is long and M x N = chunk x H is
// small); the count used fills whole rounds of the device's compute units.
constexpr int kFlceMaxSplitK = 16;
// Bytes of transposed chunk gradients and hidden states kept for one
// grad_weight GEMM: the chunks of a group are contracted in one pass, so
// grad_weight is written once per group instead of read-modify-written once
// per chunk.
constexpr size_t kFlceGroupBytes = size_t(2) << 30;

struct FlceArgs {
    const void *hidden;      // bf16 [n, H]
    const void *weight;      // bf16 [V, H]
    const int64_t *labels;   // [n]
    int64_t n, H, V, chunk;
    int64_t ignore_index;
    float eps, softcap;
    int reduction;
    const float *grad_out;   // NULL, scalar or [n]
    float *loss_tok;         // [n]
    float *loss_out;         // scalar or NULL
    void *grad_hidden;       // bf16 [n, H]
    float *grad_weight;      // fp32 [V, H], overwritten
    int64_t *counts;         // [3]
    void *workspace;
    int64_t group_chunks;    // chunks per grad_weight group (the workspace was sized for it)
    bool with_wt = true;     // the workspace holds W^T (else dH reads W in place, k-major)
    // Tile-resident backward: with lse and q (1 - p_y) of every token from the
    // stats pass, each chunk's gradient is formed in the logits GEMM's epilogue
    // (no logits stored, no losses written, counts read as given).
    const float *lse = nullptr;
    const float *q = nullptr;
    // The caller's second stream for the transposes, or null (everything on the call's stream).
    hipStream_t aux = nullptr;
};

// Stats pass of the tile-resident fused linear cross-entropy: one record per
// token and 256-column tile of Z = hidden weight^T, merged into the row outputs.
struct FlceFwdArgs {
    const void *hidden;      // bf16 [n, H]
    const void *weight;      // bf16 [V, H]
    const int64_t *labels;   // [n]
    int64_t n, H, V;
    int64_t ignore_index;
    float eps, softcap;
    int reduction;
    float *lse, *q;          // [n], required
    float *loss_tok;         // [n], required
    float *loss_out;         // scalar or NULL
    float *logp, *ent;       // [n] or NULL
    int64_t *argmax_out;     // [n] or NULL
    int64_t *counts;         // [3]
    void *workspace;         // flce_stats_bytes(n, V)
};
size_t flce_stats_bytes(int64_t n, int64_t V);
hipError_t launch_flce_forward(const FlceFwdArgs &f, hipStream_t stream);

// Offsets (bytes) of the fused-linear workspace regions.
struct FlceLayout {
    int64_t chunk;        // tokens per logits chunk
    int64_t group;        // tokens per grad_weight group (a multiple of chunk)
    int64_t ldg;          // row stride of the transposed group buffers (multiple of 8)
    size_t off_wt, off_z, off_gt, off_ht, off_part, off_ce, bytes;   // off_wt: with_wt only
};
// with_wt: room for W^T [H, V] bf16, which makes dH's GEMM read W K-contiguous
// (faster than reading W in place through transposing LDS reads, 2 H V bytes more)
FlceLayout flce_layout(int64_t n, int64_t H, int64_t V, int64_t chunk, int64_t group_chunks, bool with_wt);
// The layout a workspace of `bytes` gets: the largest grad_weight group (up to
// the default) that fits without W^T, plus W^T when there is room for it too.
// False when not even one chunk per group fits.
bool flce_plan(int64_t n, int64_t H, int64_t V, int64_t chunk, size_t bytes, int64_t *group_chunks, bool *with_wt);
// Chunks per grad_weight group that kFlceGroupBytes holds (at least 1, at most all chunks).
int64_t flce_default_group_chunks(int64_t n, int64_t H, int64_t V, int64_t chunk);
hipError_t launch_flce(const FlceArgs &f, hipStream_t stream);

}  // namespace lce
