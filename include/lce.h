/*
 * lce.h -- C ABI of the MI355X (gfx950) vocabulary cross-entropy library.
 *
 * Every entry point takes plain pointers and sizes.  "device" pointers are
 * HIP device memory owned by the caller; the library allocates no memory and
 * never synchronises the host: work is enqueued on `stream` and its outputs
 * are valid once that stream has been synchronised.  Calls on different
 * streams are independent as long as their buffers do not overlap.  The only
 * state kept between calls is the thread-local error text, and for
 * lce_ce_fwd_bwd_noalloc (callers that cannot allocate) one scratch array per
 * device; the other functions are re-entrant.
 *
 * Errors: arguments are checked before any HIP call.  A bad argument returns
 * LCE_ERR_INVALID_ARG, a valid but unsupported combination returns
 * LCE_ERR_UNSUPPORTED (the message names the constraint), a failed launch
 * returns LCE_ERR_HIP.  No exception crosses this boundary.  lce_last_error()
 * explains the most recent failure on the calling thread.
 *
 * The operations follow these pages (cited by title and section):
 *  [P1] Liger-Kernel PR "Add Megatron-LM cross-entropy integration": Summary
 *       (ignore_index=-100, label_smoothing, online softmax with the gradient
 *       written in place and no full softmax kept) and Test setup (the same
 *       operation as torch.nn.functional.cross_entropy).
 *  [P2] Megatron-LM PR "Add opt-in Liger vocab-parallel cross entropy": "What
 *       does this PR do?" (fp32 per-token losses, any upstream gradient,
 *       original argmax with smallest-index ties) and Performance (the input
 *       is consumed, so benchmarks clone it outside the timed region).
 *  [P5] Liger-Kernel PR "Add Liger Kernel support for Muse Glimmer": Summary
 *       (fused linear cross-entropy that never forms the [tokens, V] logits;
 *       token accuracy), Details/Softcap (T*tanh(x/T), the output multiplier
 *       folded into hidden by the caller) and Memory (grad_weight kept in fp32).
 */
#ifndef LCE_H
#define LCE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    LCE_OK = 0,
    LCE_ERR_INVALID_ARG = 1,
    LCE_ERR_UNSUPPORTED = 2,
    LCE_ERR_HIP = 3
} lce_status;

typedef enum { LCE_F32 = 0, LCE_BF16 = 1 } lce_dtype;

typedef enum { LCE_RED_NONE = 0, LCE_RED_MEAN = 1, LCE_RED_SUM = 2 } lce_reduction;

/*
 * Bytes of device workspace lce_ce_fwd_bwd needs for n rows of V columns
 * (256 + 16 * min(n, 4096) rounded up to a multiple of 256, plus
 * 128 * min(2 n, 512); always > 0).  The workspace holds the completion
 * counter of the final reduction, the counters the workgroups draw rows and
 * ignored-row chunks from, per-workgroup partial counts, and the records
 * through which the two workgroups of a pair exchange their half rows'
 * statistics (16-byte aligned rows of 122,888 to 153,600 bf16 or 61,444 to
 * 76,800 fp32 columns are reduced half a row per workgroup).  Each counter carries the
 * tag of the launch that set it (its dispatch id), each record word a key of
 * the launch and the step, and a reader clears a record it has taken, so the
 * workspace needs no initialisation and a call that never completed leaves
 * nothing the next call would trip over.
 */
size_t lce_ce_workspace_bytes(int64_t n, int64_t V);

/*
 * Cross-entropy forward + backward over a [n, V] logits matrix, gradient
 * written in place [P1 Summary; P2 "What does this PR do?"; P5 Details].
 *
 * For row i with label y_i (valid iff y_i != ignore_index and 0 <= y_i < V),
 * z = softcap > 0 ? softcap*tanh(x/softcap) : x, eps = label_smoothing:
 *   loss_i = LSE(z_i) - (1-eps) z_{i,y_i} - (eps/V) sum_j z_ij  (0 if invalid)
 *   dx_ij  = s_i (softmax(z_i)_j - (1-eps)[j==y_i] - eps/V) dz_ij/dx_ij (0 if invalid)
 * with s_i = g/n_valid (MEAN; 0 when n_valid == 0), g (SUM) or g_i (NONE),
 * g = grad_out (1.0 when grad_out is NULL).
 *
 *   logits_inout  device, [n, ld] row-major, dtype F32 or BF16.  Read as the
 *                 logits and overwritten with dx, rounded to nearest-even in
 *                 the same dtype.  Columns [V, ld) are neither read nor
 *                 written.  The buffer is consumed: request the argmax in
 *                 this same call if it is wanted.
 *   ld            row stride in elements, >= V.
 *   labels        device int64 [n].  Labels outside [0, V) other than
 *                 ignore_index are treated as ignored and counted in counts[2].
 *   label_smoothing  eps in [0, 1].    softcap  T >= 0 (0 = off).
 *   grad_out      device fp32: 1 element (MEAN/SUM) or [n] (NONE); NULL = 1.0.
 *   loss_tok      device fp32 [n], required: per-token losses (0 if ignored).
 *   loss_out      device fp32 scalar or NULL: mean over valid tokens (0 when
 *                 there are none) or sum.  Written as 0 for NONE.
 *   argmax_out    device int64 [n] or NULL: smallest index of the row maximum
 *                 of the raw logits, for every row (ignored rows included).
 *   counts        device int64 [3], required: {n_valid, n_correct, n_bad};
 *                 n_correct = #{valid i : argmax_i == y_i} (0 when argmax_out
 *                 is NULL).  Token accuracy = n_correct / n_valid.
 *   workspace     device scratch of at least lce_ce_workspace_bytes(n, V)
 *                 bytes, 16-byte aligned, required (NULL is
 *                 LCE_ERR_INVALID_ARG: the rows are handed out dynamically
 *                 from a counter in it).  Its contents before the call do not
 *                 matter.  Calls that share a workspace must not run
 *                 concurrently.
 * loss_tok, argmax_out, counts, workspace and loss_out must not overlap the
 * logits or each other.  n == 0 is valid (counts and loss_out become 0).
 */
lce_status lce_ce_fwd_bwd(void *logits_inout, int64_t ld, lce_dtype dtype, const int64_t *labels,
                          int64_t n, int64_t V, int64_t ignore_index, float label_smoothing,
                          float softcap, lce_reduction reduction, const float *grad_out,
                          float *loss_tok, float *loss_out, int64_t *argmax_out, int64_t *counts,
                          void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * lce_ce_fwd_bwd without a workspace argument, for callers that cannot
 * allocate device memory (code under stream capture that may not call
 * hipMalloc, tight serving loops, harnesses that forbid allocation).  Every
 * argument, output and result is that of lce_ce_fwd_bwd; the call allocates
 * nothing.  Its workspace is a file-scope device array of 131,328 bytes (room
 * for any n: lce_ce_workspace_bytes stops growing at n = 4096), one copy per
 * device, held until the process ends; the first call on a device looks up
 * that copy's address with the device current (hipGetSymbolAddress) and keeps
 * it.  The array keeps the last call's contents; its counters carry the tag of
 * the launch that set them, so nothing in it needs clearing between calls.
 * Calls that overlap on one device share that array and race: order them
 * (one stream, or events) or use lce_ce_fwd_bwd with workspaces of their own.
 */
lce_status lce_ce_fwd_bwd_noalloc(void *logits_inout, int64_t ld, lce_dtype dtype, const int64_t *labels,
                                  int64_t n, int64_t V, int64_t ignore_index, float label_smoothing,
                                  float softcap, lce_reduction reduction, const float *grad_out,
                                  float *loss_tok, float *loss_out, int64_t *argmax_out, int64_t *counts,
                                  hipStream_t stream);

/*
 * Read-only argmax sweep [P2 "What does this PR do?"; P5 Summary]: argmax_out[i]
 * = smallest index of the maximum of row i of the raw logits, for every row.
 *   logits      device [n, ld], F32 or BF16, not modified.
 *   labels      device int64 [n] or NULL.  With labels, counts = {n_valid,
 *               n_correct, n_bad}; without, counts = {0, 0, 0}.
 *   argmax_out  device int64 [n], required.   counts  device int64 [3], required.
 */
lce_status lce_ce_argmax(const void *logits, int64_t ld, lce_dtype dtype, const int64_t *labels,
                         int64_t n, int64_t V, int64_t ignore_index, int64_t *argmax_out,
                         int64_t *counts, hipStream_t stream);

/*
 * ---- split cross-entropy: shard statistics, combine, gradient -------------
 *
 * The same row operation as lce_ce_fwd_bwd in three calls, so that
 *  - the vocabulary can be split into shards (one per device in a
 *    vocabulary-parallel layout, Megatron-LM PR "Add opt-in Liger
 *    vocab-parallel cross entropy", What does this PR do?): every holder of
 *    a shard runs lce_ce_stats on it, the stats records (32 bytes per row and
 *    shard) are gathered, lce_ce_combine forms the row results, and every
 *    holder runs lce_ce_grad on its shard;
 *  - with one shard, the gradient can be deferred to a backward pass that
 *    knows the upstream gradient (lce_ce_grad), instead of being written by
 *    the forward (Liger-Kernel PR "[Megatron] Add SwiGLU integration", Known
 *    issues: an in-place forward cannot serve a reused graph);
 *  - the RL-side row outputs -- target log-probability and entropy,
 *    labs-molt PR "Enable Liger layers", Why attention, RoPE, and RL loss stay
 *    in Molt -- come out of the same sweep.
 * A shard holds the global vocabulary columns [v_offset, v_offset + shard_V)
 * of every row; labels are global.  Shard widths and ld must be multiples of
 * 8 (bf16) or 4 (fp32) elements and the shard 16-byte aligned
 * (LCE_ERR_UNSUPPORTED otherwise).  All pointers are device pointers; calls
 * are stream-ordered and never synchronise the host.
 */

/* Bytes of one shard's stats records for n rows. */
size_t lce_ce_stats_bytes(int64_t n);

/*
 * One read-only sweep of a shard [n, ld] (first shard_V columns used):
 * writes n stats records (lce_ce_stats_bytes(n) bytes) to stats.  softcap as
 * for lce_ce_fwd_bwd; the argmax is over the raw logits, first index on ties.
 */
lce_status lce_ce_stats(const void *logits, int64_t ld, lce_dtype dtype, const int64_t *labels, int64_t n,
                        int64_t shard_V, int64_t v_offset, int64_t ignore_index, float softcap, float *stats,
                        hipStream_t stream);

/*
 * Row results from the stats of `shards` shards, stored one after another
 * (shard k's records at stats + k * n * 8 floats) in ascending v_offset
 * order, the shards covering [0, V) exactly once:
 *   lse           fp32 [n], required: log sum_j exp(z_j).
 *   one_minus_py  fp32 [n] or NULL: 1 - p_y for valid rows (0 otherwise),
 *                 accumulated without the target, as lce_ce_grad needs it.
 *   loss_tok      fp32 [n] or NULL: lse - (1 - eps) z_y - (eps / V) sum_j z_j
 *                 (0 for ignored rows).
 *   loss_out      fp32 scalar or NULL (needs loss_tok): mean over valid
 *                 labels or sum; 0 for LCE_RED_NONE.
 *   logprob       fp32 [n] or NULL: log p_y = z_y - lse (0 for ignored rows).
 *   entropy       fp32 [n] or NULL: -sum_j p_j log p_j (every row).
 *   argmax_out    int64 [n] or NULL: global first-index argmax.
 *   counts        int64 [3], required: {n_valid, n_correct, n_bad}.  Its prior
 *                 contents do not matter; while the call runs, counts[1] may
 *                 hold the workgroups' completion count, replaced by n_correct
 *                 at the end, so nothing else may use it meanwhile.
 */
lce_status lce_ce_combine(const float *stats, int64_t shards, const int64_t *labels, int64_t n, int64_t V,
                          int64_t ignore_index, float label_smoothing, lce_reduction reduction, float *lse,
                          float *one_minus_py, float *loss_tok, float *loss_out, float *logprob, float *entropy,
                          int64_t *argmax_out, int64_t *counts, hipStream_t stream);

/*
 * The gradient of one shard, written in place over it (columns past shard_V
 * untouched): dx_j = s (p_j - (1 - eps)[j = y] - eps / V) dz_j/dx_j with
 * p_j = exp(z_j - lse), p_y - 1 = -one_minus_py, and s = grad_out / n_valid
 * (mean; n_valid = counts[0]), grad_out (sum) or grad_out[i] (none); grad_out
 * NULL means 1.  Ignored rows are written as zeros.  lse, one_minus_py and
 * counts come from lce_ce_combine over all shards.
 */
lce_status lce_ce_grad(void *logits_inout, int64_t ld, lce_dtype dtype, const int64_t *labels, int64_t n,
                       int64_t shard_V, int64_t v_offset, int64_t V, int64_t ignore_index, float label_smoothing,
                       float softcap, lce_reduction reduction, const float *grad_out, const float *lse,
                       const float *one_minus_py, const int64_t *counts, hipStream_t stream);

/*
 * Bytes of device workspace lce_flce_fwd_bwd uses by default (0 for invalid
 * sizes).  It holds one chunk of logits [C, V] bf16, split-K partials
 * [16, C, H] fp32, and the transposed gradients and hidden states of one
 * grad_weight group, [V + H, G] bf16: about 2 C V + 64 C H + 2 (V + H) G bytes
 * with C = min(chunk, n).  The default group G is as many chunks as 2 GiB
 * holds (at least one, at most all n tokens); grad_weight is written once per
 * group, so fewer groups mean less grad_weight traffic.  A workspace larger by
 * 2 H V bytes (rounded up to 256) also holds W^T [H, V], which the call then
 * uses so that the grad_hidden GEMM reads W K-contiguous; at the fused-linear
 * workload (4096 x 6656 x 202048) that measured no faster overall (the W^T
 * transpose costs what the GEMM saves), so the default leaves it out.
 */
size_t lce_flce_workspace_bytes(int64_t n, int64_t H, int64_t V, int64_t chunk_tokens);

/*
 * Bytes of workspace for grad_weight groups of group_chunks chunks without the
 * W^T copy (0 for invalid sizes); group_chunks = 1 is the smallest workspace
 * lce_flce_fwd_bwd accepts.
 */
size_t lce_flce_workspace_bytes_grouped(int64_t n, int64_t H, int64_t V, int64_t chunk_tokens,
                                        int64_t group_chunks);

/*
 * Fused linear cross-entropy [P5 Summary, Memory; Details/Softcap]: the loss
 * and gradients of cross-entropy over the logits Z = hidden * weight^T,
 * processed in chunks of chunk_tokens tokens so only one chunk of logits
 * exists at a time.  The row operation (ignore_index, label_smoothing,
 * softcap, reduction, grad_out) is exactly that of lce_ce_fwd_bwd applied to Z;
 * the mean's denominator counts every token's label.
 *
 *   hidden       device bf16 [n, H] row-major; any output multiplier is
 *                already folded in by the caller [P5 Details/Softcap].
 *   weight       device bf16 [V, H] row-major.
 *   labels       device int64 [n].        grad_out  as for lce_ce_fwd_bwd.
 *   loss_tok     device fp32 [n] (per-token losses of the bf16-rounded logits).
 *   loss_out     device fp32 scalar or NULL.
 *   grad_hidden  device bf16 [n, H]: dL/dhidden.
 *   grad_weight  device fp32 [V, H]: dL/dweight, overwritten (not accumulated
 *                across calls), accumulated in fp32 over the chunks [P5 Memory].
 *   counts       device int64 [3] {n_valid, 0, n_bad}.
 *   workspace    device, 256-byte aligned, clobbered (its prior contents do
 *                not matter); at least
 *                lce_flce_workspace_bytes_grouped(n, H, V, chunk_tokens, 1)
 *                bytes (LCE_ERR_INVALID_ARG otherwise).  The call uses the
 *                largest grad_weight group, up to the default one, whose
 *                layout fits workspace_bytes without W^T, and adds the W^T
 *                copy when the rest of the workspace holds it too; without
 *                it the grad_hidden GEMM reads W in place (about 15% slower
 *                for that GEMM, 2 H V bytes less workspace), which needs
 *                V * H * 2 < 4 GiB (LCE_ERR_UNSUPPORTED otherwise).
 *   stream       the stream the call is ordered on.
 *   aux_stream   NULL, or a second stream of the same device (default
 *                priority) that the bandwidth-bound transposes may run on
 *                beside the GEMMs.  The call forks it from `stream` and joins
 *                it back before returning, with three events it creates and
 *                destroys itself, so nothing it enqueues there outlives the
 *                call's work on `stream` and a captured call captures both.
 *                NULL, or a stream being captured into another graph than
 *                `stream`, runs everything on `stream`.  Calls sharing an
 *                aux_stream are ordered on it but stay correct.
 * Logits are formed in fp32 by bf16 MFMA and stored as bf16 for the row
 * kernel.  H and V must be multiples of 8 (LCE_ERR_UNSUPPORTED otherwise).
 */
lce_status lce_flce_fwd_bwd(const void *hidden, const void *weight, const int64_t *labels, int64_t n, int64_t H,
                            int64_t V, int64_t ignore_index, float label_smoothing, float softcap,
                            lce_reduction reduction, const float *grad_out, int64_t chunk_tokens, float *loss_tok,
                            float *loss_out, void *grad_hidden, float *grad_weight, int64_t *counts,
                            void *workspace, size_t workspace_bytes, hipStream_t stream, hipStream_t aux_stream);

/*
 * Tile-resident fused linear cross-entropy [P5 Summary; Details/Softcap;
 * Memory]: the logits Z = hidden * weight^T are formed tile by tile (256 x 256,
 * fp32 from bf16 MFMA) and never stored.  The forward reduces every tile to
 * per-row statistics; the backward forms the same tiles again and keeps only
 * the gradient, so the upstream gradient can arrive after the forward.  The
 * row operation is that of lce_ce_fwd_bwd applied to the fp32 logits (not the
 * bf16-rounded logits of lce_flce_fwd_bwd); the mean's denominator counts every
 * token's label.  H and V must be multiples of 8, hidden and weight 16-byte
 * aligned (LCE_ERR_UNSUPPORTED otherwise).
 */

/* Bytes of workspace lce_flce_forward needs: n * ceil(V / 256) records of 32 bytes. */
size_t lce_flce_stats_bytes(int64_t n, int64_t V);

/*
 * Forward [P5 Summary: loss and token accuracy without the logits]:
 *   hidden, weight, labels  as for lce_flce_fwd_bwd.
 *   loss_tok      fp32 [n], required; loss_out fp32 scalar or NULL (mean over
 *                 valid labels or sum; 0 for LCE_RED_NONE).
 *   lse           fp32 [n], required: log sum_j exp(z_j).
 *   one_minus_py  fp32 [n], required: 1 - p_y (0 for ignored rows), kept for
 *                 the backward.
 *   logprob, entropy  fp32 [n] or NULL: log p_y (0 for ignored rows) and
 *                 -sum_j p_j log p_j of every row.
 *   argmax_out    int64 [n] or NULL: first argmax of the raw fp32 logits.
 *   counts        int64 [3], required: {n_valid, n_correct, n_bad}; token
 *                 accuracy = n_correct / n_valid.
 *   workspace     device, 256-byte aligned, at least lce_flce_stats_bytes(n, V)
 *                 bytes (LCE_ERR_INVALID_ARG otherwise); clobbered.
 */
lce_status lce_flce_forward(const void *hidden, const void *weight, const int64_t *labels, int64_t n, int64_t H,
                            int64_t V, int64_t ignore_index, float label_smoothing, float softcap,
                            lce_reduction reduction, float *loss_tok, float *loss_out, float *lse, float *one_minus_py,
                            float *logprob, float *entropy, int64_t *argmax_out, int64_t *counts, void *workspace,
                            size_t workspace_bytes, hipStream_t stream);

/*
 * Backward: grad_hidden bf16 [n, H] and grad_weight fp32 [V, H] (overwritten)
 * from lse, one_minus_py and counts of lce_flce_forward on the same inputs and
 * options, with the upstream gradient grad_out (as for lce_ce_fwd_bwd).  Tokens
 * go in chunks of chunk_tokens; the workspace is that of lce_flce_fwd_bwd
 * (lce_flce_workspace_bytes[_grouped], the same group rule and the same 4 GiB
 * limit without W^T) and aux_stream as for lce_flce_fwd_bwd.  Nothing of the
 * forward's outputs is modified.
 */
lce_status lce_flce_backward(const void *hidden, const void *weight, const int64_t *labels, int64_t n, int64_t H,
                             int64_t V, int64_t ignore_index, float label_smoothing, float softcap,
                             lce_reduction reduction, const float *grad_out, int64_t chunk_tokens, const float *lse,
                             const float *one_minus_py, const int64_t *counts, void *grad_hidden, float *grad_weight,
                             void *workspace, size_t workspace_bytes, hipStream_t stream, hipStream_t aux_stream);

/*
 * Text of the most recent error on the calling thread ("" if none).  Valid
 * until the next lce_* call on the same thread.
 */
const char *lce_last_error(void);

/* Library ABI version (bumped on any signature change). */
int lce_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LCE_H */
