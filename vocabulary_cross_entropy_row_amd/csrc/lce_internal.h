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
    int64_t ignore_index;
    float eps;               // label smoothing
    float softcap;           // 0 = off
    int reduction;           // lce_reduction
    const float *grad_out;   // NULL = 1.0
    float *loss_tok;         // [n]
    float *loss_out;         // scalar or NULL
    int64_t *argmax_out;     // [n] or NULL
    int64_t *counts;         // [3]
    unsigned *ticket;        // completion counter (workspace)
};

// Threads per row workgroup of the register-resident path.
constexpr int kRowThreads = 1024;
// Largest number of 16-byte vectors per thread the register-resident path
// keeps (26 * 16 B = 416 B = 104 VGPRs per lane).
constexpr int kMaxVecPerThread = 26;

// Enqueue count + row kernels.  is_bf16 selects the element type.
hipError_t launch_ce_fwd_bwd(const CEArgs &a, bool is_bf16, hipStream_t stream);

// Enqueue the read-only argmax sweep (counts zeroed/filled too).
hipError_t launch_ce_argmax(const void *logits, int64_t ld, bool is_bf16, const int64_t *labels,
                            int64_t n, int64_t V, int64_t ignore_index, int64_t *argmax_out,
                            int64_t *counts, hipStream_t stream);

// Which row kernel a shape takes (exposed for tests / the bench report).
// Returns the vectors-per-thread template chosen, or 0 for the generic path.
int ce_fast_path_k(const void *logits, int64_t ld, bool is_bf16, int64_t V);

}  // namespace lce
