// C-ABI entry points (include/lce.h): argument validation, then kernel launch.
// Validation runs before any HIP call, so every argument error is reported
// without touching the device.  No exception crosses the ABI.
#include "lce.h"

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <atomic>
#include <mutex>

#include "lce_internal.h"

// The workspace of lce_ce_fwd_bwd_noalloc: room for the row kernel's workspace
// at any n (its per-workgroup part stops growing at kMaxRowGroups workgroups),
// one copy per device, held until the process ends.  Host code never uses this
// name as an address: it is a host-side stand-in for the device symbol, whose
// address on each device comes from hipGetSymbolAddress (noalloc_scratch).
constexpr size_t kNoAllocScratchBytes = lce::ce_workspace_bytes(lce::kMaxRowGroups);
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

thread_local char g_err[512] = "";

lce_status fail(lce_status st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

lce_status ok() {
    g_err[0] = '\0';
    return LCE_OK;
}

lce_status hip_status(hipError_t e, const char *what) {
    if (e == hipSuccess) return ok();
    return fail(LCE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool is_aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Checks shared by the tile-resident fused linear entry points.
lce_status check_flce_resident(const char *fn, const void *hidden, const void *weight, const int64_t *labels,
                               int64_t n, int64_t H, int64_t V, float label_smoothing, float softcap,
                               lce_reduction reduction) {
    if (n < 0) return fail(LCE_ERR_INVALID_ARG, "%s: n must be >= 0 (got %lld)", fn, (long long)n);
    if (H < 1) return fail(LCE_ERR_INVALID_ARG, "%s: H must be >= 1 (got %lld)", fn, (long long)H);
    if (V < 1) return fail(LCE_ERR_INVALID_ARG, "%s: V must be >= 1 (got %lld)", fn, (long long)V);
    if (reduction != LCE_RED_NONE && reduction != LCE_RED_MEAN && reduction != LCE_RED_SUM)
        return fail(LCE_ERR_INVALID_ARG, "%s: unknown reduction %d", fn, (int)reduction);
    if (!(label_smoothing >= 0.0f && label_smoothing <= 1.0f))
        return fail(LCE_ERR_INVALID_ARG, "%s: label_smoothing must be in [0, 1] (got %g)", fn, (double)label_smoothing);
    if (!(softcap >= 0.0f) || isinf(softcap))
        return fail(LCE_ERR_INVALID_ARG, "%s: softcap must be finite and >= 0 (got %g)", fn, (double)softcap);
    if (!weight) return fail(LCE_ERR_INVALID_ARG, "%s: weight is required", fn);
    if (n > 0 && (!hidden || !labels)) return fail(LCE_ERR_INVALID_ARG, "%s: hidden and labels are required", fn);
    if (H % 8 != 0 || V % 8 != 0)
        return fail(LCE_ERR_UNSUPPORTED, "%s: requires H and V to be multiples of 8 (16-byte bf16 rows); got H=%lld V=%lld",
                    fn, (long long)H, (long long)V);
    if ((hidden && !is_aligned(hidden, 16)) || !is_aligned(weight, 16))
        return fail(LCE_ERR_UNSUPPORTED, "%s: hidden and weight must be 16-byte aligned", fn);
    if (n > 0x7fffffffLL || V > 0x7fffffffLL / 16 || H > 0x7fffffffLL / 16 || 256ull * V * 2 >= (1ull << 32) ||
        256ull * H * 2 >= (1ull << 32))
        return fail(LCE_ERR_UNSUPPORTED, "%s: n >= 2^31 or a 256-row operand tile exceeds 4 GiB", fn);
    return LCE_OK;
}

}  // namespace

extern "C" {

int lce_abi_version(void) { return 3; }

const char *lce_last_error(void) { return g_err; }

size_t lce_ce_workspace_bytes(int64_t n, int64_t V) {
    (void)V;
    return lce::ce_workspace_bytes(n);
}

}  // extern "C"

namespace {

// Checks of lce_ce_fwd_bwd's arguments other than the workspace, in the order the
// header lists them; the call's name prefixes every message.
lce_status check_ce_args(const char *fn, const void *logits_inout, int64_t ld, lce_dtype dtype,
                         const int64_t *labels, int64_t n, int64_t V, float label_smoothing, float softcap,
                         lce_reduction reduction, const float *loss_tok, const int64_t *counts) {
    if (n < 0) return fail(LCE_ERR_INVALID_ARG, "%s: n must be >= 0 (got %lld)", fn, (long long)n);
    if (V < 1) return fail(LCE_ERR_INVALID_ARG, "%s: V must be >= 1 (got %lld)", fn, (long long)V);
    if (ld < V) return fail(LCE_ERR_INVALID_ARG, "%s: ld (%lld) must be >= V (%lld)", fn, (long long)ld, (long long)V);
    if (dtype != LCE_F32 && dtype != LCE_BF16) return fail(LCE_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, (int)dtype);
    if (reduction != LCE_RED_NONE && reduction != LCE_RED_MEAN && reduction != LCE_RED_SUM)
        return fail(LCE_ERR_INVALID_ARG, "%s: unknown reduction %d", fn, (int)reduction);
    if (!(label_smoothing >= 0.0f && label_smoothing <= 1.0f))
        return fail(LCE_ERR_INVALID_ARG, "%s: label_smoothing must be in [0, 1] (got %g)", fn, (double)label_smoothing);
    if (!(softcap >= 0.0f) || isinf(softcap))
        return fail(LCE_ERR_INVALID_ARG, "%s: softcap must be finite and >= 0 (got %g)", fn, (double)softcap);
    if (!counts) return fail(LCE_ERR_INVALID_ARG, "%s: counts is required", fn);
    if (n > 0) {
        if (!logits_inout) return fail(LCE_ERR_INVALID_ARG, "%s: logits is required", fn);
        if (!labels) return fail(LCE_ERR_INVALID_ARG, "%s: labels is required", fn);
        if (!loss_tok) return fail(LCE_ERR_INVALID_ARG, "%s: loss_tok is required", fn);
        const size_t esz = dtype == LCE_BF16 ? 2 : 4;
        if (!is_aligned(logits_inout, esz))
            return fail(LCE_ERR_INVALID_ARG, "%s: logits must be aligned to its element size", fn);
    }
    return LCE_OK;
}

lce_status launch_ce(const char *fn, void *logits_inout, int64_t ld, lce_dtype dtype, const int64_t *labels, int64_t n,
                     int64_t V, int64_t ignore_index, float label_smoothing, float softcap, lce_reduction reduction,
                     const float *grad_out, float *loss_tok, float *loss_out, int64_t *argmax_out, int64_t *counts,
                     void *workspace, hipStream_t stream) {
    if (n > 0x7fffffffLL) return fail(LCE_ERR_UNSUPPORTED, "%s: n > 2^31-1 rows is not supported", fn);
    if (V > 0x7fffffffLL / 16) return fail(LCE_ERR_UNSUPPORTED, "%s: V > 2^27 columns is not supported", fn);
    lce::CEArgs a;
    a.logits = logits_inout;
    a.ld = ld;
    a.n = n;
    a.V = V;
    a.labels = labels;
    a.count_labels = labels;
    a.count_n = n;
    a.ignore_index = ignore_index;
    a.eps = label_smoothing;
    a.softcap = softcap;
    a.reduction = static_cast<int>(reduction);
    a.grad_out = grad_out;
    a.loss_tok = loss_tok;
    a.loss_out = loss_out;
    a.argmax_out = argmax_out;
    a.counts = counts;
    a.workspace = workspace;
    char what[64];
    snprintf(what, sizeof what, "%s launch", fn);
    return hip_status(lce::launch_ce_fwd_bwd(a, dtype == LCE_BF16, stream), what);
}

// Device address of `scratch` on each device, looked up by the first
// lce_ce_fwd_bwd_noalloc call on that device (with the device current).
constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;   // taken only until a device's address is known

lce_status noalloc_scratch(const char *fn, hipStream_t stream, void **out) {
    int dev = -1;
    hipError_t e = hipStreamGetDevice(stream, &dev);
    if (e != hipSuccess) return hip_status(e, "lce_ce_fwd_bwd_noalloc: hipStreamGetDevice");
    if (dev < 0 || dev >= kMaxDevices)
        return fail(LCE_ERR_UNSUPPORTED, "%s: device %d is beyond the %d devices the scratch table holds", fn, dev,
                    kMaxDevices);
    void *p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch[dev].load(std::memory_order_acquire);
        if (!p) {
            int cur = -1;
            if ((e = hipGetDevice(&cur)) != hipSuccess) return hip_status(e, "lce_ce_fwd_bwd_noalloc: hipGetDevice");
            if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess)
                return hip_status(e, "lce_ce_fwd_bwd_noalloc: hipSetDevice");
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            const hipError_t back = cur != dev ? hipSetDevice(cur) : hipSuccess;
            if (e != hipSuccess) return hip_status(e, "lce_ce_fwd_bwd_noalloc: hipGetSymbolAddress");
            if (back != hipSuccess) return hip_status(back, "lce_ce_fwd_bwd_noalloc: hipSetDevice");
            if (!p) return fail(LCE_ERR_HIP, "%s: hipGetSymbolAddress gave a null address", fn);
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return LCE_OK;
}

}  // namespace

extern "C" {

lce_status lce_ce_fwd_bwd(void *logits_inout, int64_t ld, lce_dtype dtype, const int64_t *labels, int64_t n,
                          int64_t V, int64_t ignore_index, float label_smoothing, float softcap,
                          lce_reduction reduction, const float *grad_out, float *loss_tok, float *loss_out,
                          int64_t *argmax_out, int64_t *counts, void *workspace, size_t workspace_bytes,
                          hipStream_t stream) {
    const char *fn = "lce_ce_fwd_bwd";
    lce_status st = check_ce_args(fn, logits_inout, ld, dtype, labels, n, V, label_smoothing, softcap, reduction,
                                  loss_tok, counts);
    if (st != LCE_OK) return st;
    if (!workspace) return fail(LCE_ERR_INVALID_ARG, "%s: workspace is required", fn);
    if (workspace_bytes < lce_ce_workspace_bytes(n, V))
        return fail(LCE_ERR_INVALID_ARG, "%s: workspace_bytes %zu < required %zu", fn, workspace_bytes,
                    lce_ce_workspace_bytes(n, V));
    if (!is_aligned(workspace, 16)) return fail(LCE_ERR_INVALID_ARG, "%s: workspace must be 16-byte aligned", fn);
    return launch_ce(fn, logits_inout, ld, dtype, labels, n, V, ignore_index, label_smoothing, softcap, reduction,
                     grad_out, loss_tok, loss_out, argmax_out, counts, workspace, stream);
}

lce_status lce_ce_fwd_bwd_noalloc(void *logits_inout, int64_t ld, lce_dtype dtype, const int64_t *labels, int64_t n,
                                  int64_t V, int64_t ignore_index, float label_smoothing, float softcap,
                                  lce_reduction reduction, const float *grad_out, float *loss_tok, float *loss_out,
                                  int64_t *argmax_out, int64_t *counts, hipStream_t stream) {
    const char *fn = "lce_ce_fwd_bwd_noalloc";
    lce_status st = check_ce_args(fn, logits_inout, ld, dtype, labels, n, V, label_smoothing, softcap, reduction,
                                  loss_tok, counts);
    if (st != LCE_OK) return st;
    if (lce_ce_workspace_bytes(n, V) > kNoAllocScratchBytes)
        return fail(LCE_ERR_UNSUPPORTED, "%s: needs %zu bytes of scratch, more than the %zu it holds", fn,
                    lce_ce_workspace_bytes(n, V), kNoAllocScratchBytes);
    void *ws = nullptr;
    if ((st = noalloc_scratch(fn, stream, &ws)) != LCE_OK) return st;
    return launch_ce(fn, logits_inout, ld, dtype, labels, n, V, ignore_index, label_smoothing, softcap, reduction,
                     grad_out, loss_tok, loss_out, argmax_out, counts, ws, stream);
}

lce_status lce_ce_argmax(const void *logits, int64_t ld, lce_dtype dtype, const int64_t *labels, int64_t n,
                         int64_t V, int64_t ignore_index, int64_t *argmax_out, int64_t *counts,
                         hipStream_t stream) {
    if (n < 0) return fail(LCE_ERR_INVALID_ARG, "lce_ce_argmax: n must be >= 0 (got %lld)", (long long)n);
    if (V < 1) return fail(LCE_ERR_INVALID_ARG, "lce_ce_argmax: V must be >= 1 (got %lld)", (long long)V);
    if (ld < V) return fail(LCE_ERR_INVALID_ARG, "lce_ce_argmax: ld (%lld) must be >= V (%lld)", (long long)ld,
                            (long long)V);
    if (dtype != LCE_F32 && dtype != LCE_BF16)
        return fail(LCE_ERR_INVALID_ARG, "lce_ce_argmax: unknown dtype %d", (int)dtype);
    if (!counts) return fail(LCE_ERR_INVALID_ARG, "lce_ce_argmax: counts is required");
    if (n > 0) {
        if (!logits) return fail(LCE_ERR_INVALID_ARG, "lce_ce_argmax: logits is required");
        if (!argmax_out) return fail(LCE_ERR_INVALID_ARG, "lce_ce_argmax: argmax_out is required");
        const size_t esz = dtype == LCE_BF16 ? 2 : 4;
        if (!is_aligned(logits, esz))
            return fail(LCE_ERR_INVALID_ARG, "lce_ce_argmax: logits must be aligned to its element size");
    }
    if (n > 0x7fffffffLL) return fail(LCE_ERR_UNSUPPORTED, "lce_ce_argmax: n > 2^31-1 rows is not supported");
    if (V > 0x7fffffffLL / 16) return fail(LCE_ERR_UNSUPPORTED, "lce_ce_argmax: V > 2^27 columns is not supported");
    return hip_status(lce::launch_ce_argmax(logits, ld, dtype == LCE_BF16, labels, n, V, ignore_index, argmax_out,
                                            counts, stream),
                      "lce_ce_argmax launch");
}

// shared checks of a logits shard [n, Vs] with row stride ld
static lce_status check_shard(const char *fn, const void *logits, int64_t ld, lce_dtype dtype, const int64_t *labels,
                              int64_t n, int64_t Vs, int64_t v0) {
    if (n < 0) return fail(LCE_ERR_INVALID_ARG, "%s: n must be >= 0 (got %lld)", fn, (long long)n);
    if (Vs < 1) return fail(LCE_ERR_INVALID_ARG, "%s: the shard width must be >= 1 (got %lld)", fn, (long long)Vs);
    if (v0 < 0) return fail(LCE_ERR_INVALID_ARG, "%s: v_offset must be >= 0 (got %lld)", fn, (long long)v0);
    if (ld < Vs) return fail(LCE_ERR_INVALID_ARG, "%s: ld (%lld) must be >= the shard width (%lld)", fn,
                             (long long)ld, (long long)Vs);
    if (dtype != LCE_F32 && dtype != LCE_BF16) return fail(LCE_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, (int)dtype);
    if (n > 0 && (!logits || !labels)) return fail(LCE_ERR_INVALID_ARG, "%s: logits and labels are required", fn);
    const int64_t E = dtype == LCE_BF16 ? 8 : 4;
    if (Vs % E != 0 || ld % E != 0 || (logits && !is_aligned(logits, 16)))
        return fail(LCE_ERR_UNSUPPORTED,
                    "%s: requires 16-byte rows (shard width and ld multiples of %lld elements, 16-byte aligned logits)",
                    fn, (long long)E);
    if (n > 0x7fffffffLL) return fail(LCE_ERR_UNSUPPORTED, "%s: n > 2^31-1 rows is not supported", fn);
    if (v0 + Vs > 0x7fffffffLL || Vs * (dtype == LCE_BF16 ? 2 : 4) >= (1ll << 32))
        return fail(LCE_ERR_UNSUPPORTED, "%s: vocabulary indexes must fit 31 bits and a shard row 4 GiB", fn);
    return LCE_OK;
}

size_t lce_ce_stats_bytes(int64_t n) { return n < 0 ? 0 : static_cast<size_t>(n) * lce::kStatsFloats * sizeof(float); }

lce_status lce_ce_stats(const void *logits, int64_t ld, lce_dtype dtype, const int64_t *labels, int64_t n,
                        int64_t shard_V, int64_t v_offset, int64_t ignore_index, float softcap, float *stats,
                        hipStream_t stream) {
    const char *fn = "lce_ce_stats";
    lce_status st = check_shard(fn, logits, ld, dtype, labels, n, shard_V, v_offset);
    if (st != LCE_OK) return st;
    if (!(softcap >= 0.0f) || isinf(softcap))
        return fail(LCE_ERR_INVALID_ARG, "%s: softcap must be finite and >= 0 (got %g)", fn, (double)softcap);
    if (n > 0 && !stats) return fail(LCE_ERR_INVALID_ARG, "%s: stats is required", fn);
    return hip_status(lce::launch_ce_stats(logits, ld, dtype == LCE_BF16, labels, n, shard_V, v_offset, ignore_index,
                                           softcap, stats, stream),
                      "lce_ce_stats launch");
}

lce_status lce_ce_combine(const float *stats, int64_t shards, const int64_t *labels, int64_t n, int64_t V,
                          int64_t ignore_index, float label_smoothing, lce_reduction reduction, float *lse,
                          float *one_minus_py, float *loss_tok, float *loss_out, float *logprob, float *entropy,
                          int64_t *argmax_out, int64_t *counts, hipStream_t stream) {
    const char *fn = "lce_ce_combine";
    if (n < 0) return fail(LCE_ERR_INVALID_ARG, "%s: n must be >= 0 (got %lld)", fn, (long long)n);
    if (V < 1) return fail(LCE_ERR_INVALID_ARG, "%s: V must be >= 1 (got %lld)", fn, (long long)V);
    if (shards < 1) return fail(LCE_ERR_INVALID_ARG, "%s: shards must be >= 1 (got %lld)", fn, (long long)shards);
    if (reduction != LCE_RED_NONE && reduction != LCE_RED_MEAN && reduction != LCE_RED_SUM)
        return fail(LCE_ERR_INVALID_ARG, "%s: unknown reduction %d", fn, (int)reduction);
    if (!(label_smoothing >= 0.0f && label_smoothing <= 1.0f))
        return fail(LCE_ERR_INVALID_ARG, "%s: label_smoothing must be in [0, 1] (got %g)", fn, (double)label_smoothing);
    if (!counts) return fail(LCE_ERR_INVALID_ARG, "%s: counts is required", fn);
    if (n > 0 && (!stats || !labels || !lse))
        return fail(LCE_ERR_INVALID_ARG, "%s: stats, labels and lse are required", fn);
    if (n > 0 && loss_out && !loss_tok) return fail(LCE_ERR_INVALID_ARG, "%s: loss_out needs loss_tok", fn);
    if (n > 0x7fffffffLL) return fail(LCE_ERR_UNSUPPORTED, "%s: n > 2^31-1 rows is not supported", fn);
    return hip_status(lce::launch_ce_combine(stats, shards, n, 1, labels, n, V, ignore_index, label_smoothing,
                                             static_cast<int>(reduction), lse, one_minus_py, loss_tok, loss_out,
                                             logprob, entropy, argmax_out, counts, stream),
                      "lce_ce_combine launch");
}

lce_status lce_ce_grad(void *logits_inout, int64_t ld, lce_dtype dtype, const int64_t *labels, int64_t n,
                       int64_t shard_V, int64_t v_offset, int64_t V, int64_t ignore_index, float label_smoothing,
                       float softcap, lce_reduction reduction, const float *grad_out, const float *lse,
                       const float *one_minus_py, const int64_t *counts, hipStream_t stream) {
    const char *fn = "lce_ce_grad";
    lce_status st = check_shard(fn, logits_inout, ld, dtype, labels, n, shard_V, v_offset);
    if (st != LCE_OK) return st;
    if (V < 1 || v_offset + shard_V > V)
        return fail(LCE_ERR_INVALID_ARG, "%s: the shard [%lld, %lld) must lie inside [0, V = %lld)", fn,
                    (long long)v_offset, (long long)(v_offset + shard_V), (long long)V);
    if (reduction != LCE_RED_NONE && reduction != LCE_RED_MEAN && reduction != LCE_RED_SUM)
        return fail(LCE_ERR_INVALID_ARG, "%s: unknown reduction %d", fn, (int)reduction);
    if (!(label_smoothing >= 0.0f && label_smoothing <= 1.0f))
        return fail(LCE_ERR_INVALID_ARG, "%s: label_smoothing must be in [0, 1] (got %g)", fn, (double)label_smoothing);
    if (!(softcap >= 0.0f) || isinf(softcap))
        return fail(LCE_ERR_INVALID_ARG, "%s: softcap must be finite and >= 0 (got %g)", fn, (double)softcap);
    if (n > 0 && (!lse || !one_minus_py || !counts))
        return fail(LCE_ERR_INVALID_ARG, "%s: lse, one_minus_py and counts are required", fn);
    return hip_status(lce::launch_ce_grad(logits_inout, ld, dtype == LCE_BF16, labels, n, shard_V, v_offset, V,
                                          ignore_index, label_smoothing, softcap, static_cast<int>(reduction),
                                          grad_out, lse, one_minus_py, counts, stream),
                      "lce_ce_grad launch");
}

size_t lce_flce_workspace_bytes(int64_t n, int64_t H, int64_t V, int64_t chunk_tokens) {
    if (n < 0 || H < 1 || V < 1 || chunk_tokens < 1) return 0;
    return lce::flce_layout(n, H, V, chunk_tokens, lce::flce_default_group_chunks(n, H, V, chunk_tokens), false).bytes;
}

size_t lce_flce_workspace_bytes_grouped(int64_t n, int64_t H, int64_t V, int64_t chunk_tokens, int64_t group_chunks) {
    if (n < 0 || H < 1 || V < 1 || chunk_tokens < 1 || group_chunks < 1) return 0;
    return lce::flce_layout(n, H, V, chunk_tokens, group_chunks, false).bytes;
}

lce_status lce_flce_fwd_bwd(const void *hidden, const void *weight, const int64_t *labels, int64_t n, int64_t H,
                            int64_t V, int64_t ignore_index, float label_smoothing, float softcap,
                            lce_reduction reduction, const float *grad_out, int64_t chunk_tokens, float *loss_tok,
                            float *loss_out, void *grad_hidden, float *grad_weight, int64_t *counts, void *workspace,
                            size_t workspace_bytes, hipStream_t stream, hipStream_t aux_stream) {
    const char *fn = "lce_flce_fwd_bwd";
    if (n < 0) return fail(LCE_ERR_INVALID_ARG, "%s: n must be >= 0 (got %lld)", fn, (long long)n);
    if (H < 1) return fail(LCE_ERR_INVALID_ARG, "%s: H must be >= 1 (got %lld)", fn, (long long)H);
    if (V < 1) return fail(LCE_ERR_INVALID_ARG, "%s: V must be >= 1 (got %lld)", fn, (long long)V);
    if (chunk_tokens < 1) return fail(LCE_ERR_INVALID_ARG, "%s: chunk_tokens must be >= 1", fn);
    if (reduction != LCE_RED_NONE && reduction != LCE_RED_MEAN && reduction != LCE_RED_SUM)
        return fail(LCE_ERR_INVALID_ARG, "%s: unknown reduction %d", fn, (int)reduction);
    if (!(label_smoothing >= 0.0f && label_smoothing <= 1.0f))
        return fail(LCE_ERR_INVALID_ARG, "%s: label_smoothing must be in [0, 1] (got %g)", fn, (double)label_smoothing);
    if (!(softcap >= 0.0f) || isinf(softcap))
        return fail(LCE_ERR_INVALID_ARG, "%s: softcap must be finite and >= 0 (got %g)", fn, (double)softcap);
    if (!weight || !grad_weight || !counts || !workspace)
        return fail(LCE_ERR_INVALID_ARG, "%s: weight, grad_weight, counts and workspace are required", fn);
    if (n > 0 && (!hidden || !labels || !loss_tok || !grad_hidden))
        return fail(LCE_ERR_INVALID_ARG, "%s: hidden, labels, loss_tok and grad_hidden are required", fn);
    // the largest grad_weight group (up to the default) whose layout fits the workspace
    int64_t group = 1;
    bool with_wt = false;
    const bool fits = lce::flce_plan(n, H, V, chunk_tokens, workspace_bytes, &group, &with_wt);
    const size_t need = lce::flce_layout(n, H, V, chunk_tokens, 1, false).bytes;
    if (!fits)
        return fail(LCE_ERR_INVALID_ARG, "%s: workspace_bytes %zu < minimum %zu", fn, workspace_bytes, need);
    if (!is_aligned(workspace, 256)) return fail(LCE_ERR_INVALID_ARG, "%s: workspace must be 256-byte aligned", fn);
    if (H % 8 != 0 || V % 8 != 0)
        return fail(LCE_ERR_UNSUPPORTED, "%s: requires H and V to be multiples of 8 (16-byte bf16 rows); got H=%lld V=%lld",
                    fn, (long long)H, (long long)V);
    if ((hidden && !is_aligned(hidden, 16)) || !is_aligned(weight, 16) || (grad_hidden && !is_aligned(grad_hidden, 16)) ||
        !is_aligned(grad_weight, 16))
        return fail(LCE_ERR_UNSUPPORTED, "%s: hidden, weight, grad_hidden and grad_weight must be 16-byte aligned", fn);
    const int64_t C = chunk_tokens < n ? chunk_tokens : n;
    if (V > 0x7fffffffLL / 16 || H > 0x7fffffffLL / 16 || C > 0x7fffffffLL / 16 ||
        static_cast<unsigned long long>(C) * V * 2 >= (1ull << 32) || 256ull * V * 2 >= (1ull << 32) ||
        256ull * H * 2 >= (1ull << 32))
        return fail(LCE_ERR_UNSUPPORTED, "%s: a chunk of logits or a 256-row operand tile exceeds 4 GiB", fn);
    if (!with_wt && n > 0 && static_cast<unsigned long long>(V) * H * 2 >= (1ull << 32))
        return fail(LCE_ERR_UNSUPPORTED,
                    "%s: without room for W^T in the workspace the grad_hidden GEMM reads the weight in place, "
                    "which needs V * H * 2 < 4 GiB (V=%lld H=%lld); pass lce_flce_workspace_bytes() bytes", fn,
                    (long long)V, (long long)H);
    lce::FlceArgs f;
    f.hidden = hidden;
    f.weight = weight;
    f.labels = labels;
    f.n = n;
    f.H = H;
    f.V = V;
    f.chunk = chunk_tokens;
    f.ignore_index = ignore_index;
    f.eps = label_smoothing;
    f.softcap = softcap;
    f.reduction = static_cast<int>(reduction);
    f.grad_out = grad_out;
    f.loss_tok = loss_tok;
    f.loss_out = loss_out;
    f.grad_hidden = grad_hidden;
    f.grad_weight = grad_weight;
    f.counts = counts;
    f.workspace = workspace;
    f.group_chunks = group;
    f.with_wt = with_wt;
    f.aux = aux_stream;
    return hip_status(lce::launch_flce(f, stream), "lce_flce_fwd_bwd launch");
}

size_t lce_flce_stats_bytes(int64_t n, int64_t V) {
    if (n < 0 || V < 1) return 0;
    return lce::flce_stats_bytes(n, V);
}

lce_status lce_flce_forward(const void *hidden, const void *weight, const int64_t *labels, int64_t n, int64_t H,
                            int64_t V, int64_t ignore_index, float label_smoothing, float softcap,
                            lce_reduction reduction, float *loss_tok, float *loss_out, float *lse, float *one_minus_py,
                            float *logprob, float *entropy, int64_t *argmax_out, int64_t *counts, void *workspace,
                            size_t workspace_bytes, hipStream_t stream) {
    const char *fn = "lce_flce_forward";
    lce_status st = check_flce_resident(fn, hidden, weight, labels, n, H, V, label_smoothing, softcap, reduction);
    if (st != LCE_OK) return st;
    if (!counts) return fail(LCE_ERR_INVALID_ARG, "%s: counts is required", fn);
    if (n > 0 && (!loss_tok || !lse || !one_minus_py))
        return fail(LCE_ERR_INVALID_ARG, "%s: loss_tok, lse and one_minus_py are required", fn);
    const size_t need = lce::flce_stats_bytes(n, V);
    if (n > 0 && (!workspace || workspace_bytes < need))
        return fail(LCE_ERR_INVALID_ARG, "%s: workspace_bytes %zu < minimum %zu", fn, workspace_bytes, need);
    if (n > 0 && !is_aligned(workspace, 256))
        return fail(LCE_ERR_INVALID_ARG, "%s: workspace must be 256-byte aligned", fn);
    lce::FlceFwdArgs f;
    f.hidden = hidden;
    f.weight = weight;
    f.labels = labels;
    f.n = n;
    f.H = H;
    f.V = V;
    f.ignore_index = ignore_index;
    f.eps = label_smoothing;
    f.softcap = softcap;
    f.reduction = static_cast<int>(reduction);
    f.lse = lse;
    f.q = one_minus_py;
    f.loss_tok = loss_tok;
    f.loss_out = loss_out;
    f.logp = logprob;
    f.ent = entropy;
    f.argmax_out = argmax_out;
    f.counts = counts;
    f.workspace = workspace;
    return hip_status(lce::launch_flce_forward(f, stream), "lce_flce_forward launch");
}

lce_status lce_flce_backward(const void *hidden, const void *weight, const int64_t *labels, int64_t n, int64_t H,
                             int64_t V, int64_t ignore_index, float label_smoothing, float softcap,
                             lce_reduction reduction, const float *grad_out, int64_t chunk_tokens, const float *lse,
                             const float *one_minus_py, const int64_t *counts, void *grad_hidden, float *grad_weight,
                             void *workspace, size_t workspace_bytes, hipStream_t stream, hipStream_t aux_stream) {
    const char *fn = "lce_flce_backward";
    lce_status st = check_flce_resident(fn, hidden, weight, labels, n, H, V, label_smoothing, softcap, reduction);
    if (st != LCE_OK) return st;
    if (chunk_tokens < 1) return fail(LCE_ERR_INVALID_ARG, "%s: chunk_tokens must be >= 1", fn);
    if (!grad_weight || !counts || !workspace)
        return fail(LCE_ERR_INVALID_ARG, "%s: grad_weight, counts and workspace are required", fn);
    if (n > 0 && (!grad_hidden || !lse || !one_minus_py))
        return fail(LCE_ERR_INVALID_ARG, "%s: grad_hidden, lse and one_minus_py are required", fn);
    if ((grad_hidden && !is_aligned(grad_hidden, 16)) || !is_aligned(grad_weight, 16))
        return fail(LCE_ERR_UNSUPPORTED, "%s: grad_hidden and grad_weight must be 16-byte aligned", fn);
    int64_t group = 1;
    bool with_wt = false;
    const bool fits = lce::flce_plan(n, H, V, chunk_tokens, workspace_bytes, &group, &with_wt);
    const size_t need = lce::flce_layout(n, H, V, chunk_tokens, 1, false).bytes;
    if (!fits)
        return fail(LCE_ERR_INVALID_ARG, "%s: workspace_bytes %zu < minimum %zu", fn, workspace_bytes, need);
    if (!is_aligned(workspace, 256)) return fail(LCE_ERR_INVALID_ARG, "%s: workspace must be 256-byte aligned", fn);
    const int64_t C = chunk_tokens < n ? chunk_tokens : n;
    if (C > 0x7fffffffLL / 16 || static_cast<unsigned long long>(C) * V * 2 >= (1ull << 32))
        return fail(LCE_ERR_UNSUPPORTED, "%s: a chunk of gradients exceeds 4 GiB", fn);
    if (!with_wt && n > 0 && static_cast<unsigned long long>(V) * H * 2 >= (1ull << 32))
        return fail(LCE_ERR_UNSUPPORTED,
                    "%s: without room for W^T in the workspace the grad_hidden GEMM reads the weight in place, "
                    "which needs V * H * 2 < 4 GiB (V=%lld H=%lld); pass lce_flce_workspace_bytes() bytes", fn,
                    (long long)V, (long long)H);
    lce::FlceArgs f;
    f.hidden = hidden;
    f.weight = weight;
    f.labels = labels;
    f.n = n;
    f.H = H;
    f.V = V;
    f.chunk = chunk_tokens;
    f.ignore_index = ignore_index;
    f.eps = label_smoothing;
    f.softcap = softcap;
    f.reduction = static_cast<int>(reduction);
    f.grad_out = grad_out;
    f.loss_tok = nullptr;
    f.loss_out = nullptr;
    f.grad_hidden = grad_hidden;
    f.grad_weight = grad_weight;
    f.counts = const_cast<int64_t *>(counts);   // read only on this path
    f.workspace = workspace;
    f.group_chunks = group;
    f.with_wt = with_wt;
    f.lse = lse;
    f.q = one_minus_py;
    f.aux = aux_stream;
    return hip_status(lce::launch_flce(f, stream), "lce_flce_backward launch");
}

}  // extern "C"
