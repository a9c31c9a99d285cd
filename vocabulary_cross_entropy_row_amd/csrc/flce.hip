// Fused linear cross-entropy for gfx950 (Liger-Kernel PR "Add Liger Kernel
// support for Muse Glimmer": Summary -- the loss of hidden x weight^T without
// forming the [tokens, V] logits; Memory -- grad_weight accumulated in fp32;
// Details/Softcap -- T tanh(x / T), output multiplier already folded into
// hidden by the caller).
//
// The tokens are processed in chunks of `chunk` rows.  Per chunk c:
//   Z_c  = H_c W^T           bf16 MFMA GEMM, fp32 accumulate, stored bf16 [chunk, V]
//   G_c  = CE(Z_c)           the resident row kernel, in place, with the mean
//                            scale of all n tokens; per-token losses
//   dH_c = G_c W             split-K MFMA GEMM into fp32 partials, folded to bf16;
//                            from W^T (transposed once per call) when the
//                            workspace holds it, else from W in place (k-major
//                            B operand, transposing LDS reads: 2 H V bytes less
//                            workspace, ~15% slower GEMM)
//   G_c^T, H_c^T             appended to the current group's transposed buffers
// and once per group of chunks (as many as kFlceGroupBytes holds):
//   dW (+)= G_g^T H_g        MFMA GEMM over the group's tokens, fp32 (written
//                            by the first group, read-modify-written by later ones)
// The dW GEMM runs in the "A K-contiguous, B K-contiguous" form, so H_c^T and
// G_c^T come from a bandwidth-bound transpose (reading both dW operands
// k-major measured 15% slower than transposing them).  Only one chunk of
// logits exists at a time.
#include <hip/hip_runtime.h>
#include <algorithm>
#include <stdint.h>

#include "ce_device.h"
#include "gemm_mfma.h"
#include "lce_internal.h"

namespace lce {
namespace {

using gemm::GemmArgs;

// out[c][r] = in[r][c] for a [rows, cols] bf16 matrix (strides in elements);
// output columns [rows, rows_pad) are written as zeros, so a GEMM may run its
// K loop over whole 8-element chunks.  A workgroup moves a tile of kTrRows input
// rows x 64 columns through LDS: each 16-byte chunk of an input row lands in LDS
// with one 16-byte write, in slot (chunk ^ (row / 8) % 8) of its 128-byte LDS
// row, so the writes of a wave cover 1 KB without conflicts and the 2-byte
// reads of one output chunk (eight input rows, one column) from eight lanes
// with different row groups fall in different banks.  16-byte global loads and
// stores where aligned; each thread has four loads in flight.
constexpr int kTrRows = 128;
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const uint16_t *in, int64_t ld_in, uint16_t *out,
                                                             int64_t ld_out, int rows, int rows_pad, int cols) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    constexpr int kPer = kTrRows * 8 / 256;   // 16-byte chunks per thread, each way
    __shared__ __align__(16) uint16_t tile[kTrRows * 64];
    const int r0 = blockIdx.y * kTrRows, c0 = blockIdx.x * 64;
    const int t = threadIdx.x;
    const bool vin = ((ld_in & 7) == 0) && ((reinterpret_cast<uintptr_t>(in) & 15) == 0);
    const bool vout = ((ld_out & 7) == 0) && ((reinterpret_cast<uintptr_t>(out) & 15) == 0);
    u32x4 q[kPer];
    if (vin && r0 + kTrRows <= rows && c0 + 64 <= cols) {   // interior tile: no checks, every load in flight
#pragma unroll
        for (int h = 0; h < kPer; ++h) {   // chunk ch of input row r
            const int idx = t + h * 256, r = idx >> 3, ch = idx & 7;
            q[h] = *reinterpret_cast<const u32x4 *>(in + static_cast<int64_t>(r0 + r) * ld_in + c0 + ch * 8);
        }
    } else {
#pragma unroll
        for (int h = 0; h < kPer; ++h) {
            const int idx = t + h * 256, r = idx >> 3, ch = idx & 7;
            const int gr = r0 + r, gc = c0 + ch * 8;
            if (vin && gr < rows && gc + 7 < cols) {
                q[h] = *reinterpret_cast<const u32x4 *>(in + static_cast<int64_t>(gr) * ld_in + gc);
            } else {
                uint16_t v[8];
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    v[e] = (gr < rows && gc + e < cols) ? in[static_cast<int64_t>(gr) * ld_in + gc + e] : uint16_t(0);
#pragma unroll
                for (int w = 0; w < 4; ++w) q[h][w] = v[2 * w] | (static_cast<uint32_t>(v[2 * w + 1]) << 16);
            }
        }
    }
#pragma unroll
    for (int h = 0; h < kPer; ++h) {
        const int idx = t + h * 256, r = idx >> 3, ch = idx & 7;
        *reinterpret_cast<u32x4 *>(tile + r * 64 + ((ch ^ (r >> 3)) & 7) * 8) = q[h];
    }
    __syncthreads();
    // output row orow (= input column c0 + orow), chunk ch of eight input rows; a wave
    // takes eight output rows and eight chunks of each (128 contiguous bytes per row)
    const bool full_out = vout && r0 + kTrRows <= rows_pad && c0 + 64 <= cols;
#pragma unroll
    for (int h = 0; h < kPer; ++h) {
        const int idx = t + h * 256;
        const int orow = (idx >> 3) & 63, ch = (idx & 7) + 8 * (idx >> 9);
        const int gc = c0 + orow, gr = r0 + ch * 8;
        const uint16_t *src = tile + ch * 8 * 64 + (((orow >> 3) ^ ch) & 7) * 8 + (orow & 7);
        uint16_t v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = src[e * 64];
        uint16_t *dst = out + static_cast<int64_t>(gc) * ld_out + gr;
        if (full_out || (vout && gc < cols && gr + 7 < rows_pad)) {
            u32x4 o;
#pragma unroll
            for (int w = 0; w < 4; ++w) o[w] = v[2 * w] | (static_cast<uint32_t>(v[2 * w + 1]) << 16);
            *reinterpret_cast<u32x4 *>(dst) = o;
        } else if (gc < cols) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (gr + e < rows_pad) dst[e] = v[e];
        }
    }
}

// out[m][n] = bf16(sum_s part[s][m][n])   (part rows of stride N, splits of stride split_stride)
__global__ __launch_bounds__(256) void splitk_fold_kernel(const float *part, int64_t split_stride, int splits,
                                                          uint16_t *out, int64_t ld_out, int M, int N) {
    // four consecutive columns per thread (N is a multiple of 8); the splits are
    // added in index order, two loads in flight
    typedef __bf16 bf4 __attribute__((ext_vector_type(4)));
    const int64_t total4 = static_cast<int64_t>(M) * N / 4;
    for (int64_t q = blockIdx.x * 256ll + threadIdx.x; q < total4; q += static_cast<int64_t>(gridDim.x) * 256) {
        const int64_t i = q * 4;
        float4 s = *reinterpret_cast<const float4 *>(part + i);
        int k = 1;
        for (; k + 1 < splits; k += 2) {
            const float4 a = *reinterpret_cast<const float4 *>(part + k * split_stride + i);
            const float4 b = *reinterpret_cast<const float4 *>(part + (k + 1) * split_stride + i);
            s.x = (s.x + a.x) + b.x;
            s.y = (s.y + a.y) + b.y;
            s.z = (s.z + a.z) + b.z;
            s.w = (s.w + a.w) + b.w;
        }
        if (k < splits) {
            const float4 a = *reinterpret_cast<const float4 *>(part + k * split_stride + i);
            s.x += a.x;
            s.y += a.y;
            s.z += a.z;
            s.w += a.w;
        }
        const int64_t m = i / N, n = i - m * N;
        // converted straight into the store (RNE)
        *reinterpret_cast<bf4 *>(reinterpret_cast<__bf16 *>(out) + m * ld_out + n) =
            (bf4){static_cast<__bf16>(s.x), static_cast<__bf16>(s.y), static_cast<__bf16>(s.z), static_cast<__bf16>(s.w)};
    }
}

// loss_out from all per-token losses (fixed-order fp64 sum): mean over the
// valid count, or sum; 0 for 'none'
__global__ __launch_bounds__(1024) void loss_fold_kernel(const float *loss_tok, int64_t n, const int64_t *counts,
                                                         int reduction, float *loss_out) {
    __shared__ double sh[16];
    double acc = 0.0;
    for (int64_t i = threadIdx.x; i < n; i += 1024) acc += static_cast<double>(loss_tok[i]);
    acc = dev::wave_sum_d(acc);
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        double tot = 0.0;
        for (int w = 0; w < 16; ++w) tot += sh[w];
        float out = 0.0f;
        if (reduction == 1) out = counts[0] > 0 ? static_cast<float>(tot / static_cast<double>(counts[0])) : 0.0f;
        else if (reduction == 2) out = static_cast<float>(tot);
        *loss_out = out;
    }
}

__global__ __launch_bounds__(256) void fill_zero_f32_kernel(float *p, int64_t n) {
    for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n; i += static_cast<int64_t>(gridDim.x) * 256) p[i] = 0.0f;
}

int ceil_div(int64_t a, int64_t b) { return static_cast<int>((a + b - 1) / b); }

hipError_t transpose(const void *in, int64_t ld_in, void *out, int64_t ld_out, int rows, int rows_pad, int cols,
                     hipStream_t st) {
    if (rows_pad <= 0 || cols <= 0) return hipSuccess;
    const dim3 grid(ceil_div(cols, 64), ceil_div(rows_pad, kTrRows));
    hipLaunchKernelGGL(transpose_bf16_kernel, grid, dim3(256), 0, st, static_cast<const uint16_t *>(in), ld_in,
                       static_cast<uint16_t *>(out), ld_out, rows, rows_pad, cols);
    return hipGetLastError();
}

// The K-contiguous GEMMs request B two steps ahead (five LDS slots, 160 KB).  The GEMM that
// reads B k-major keeps two stages (128 KB): it runs while the gradient transposes of the
// second stream fill the rest of each CU's LDS.
template <int MODE, bool SOFTCAP = false, bool B_KN = false>
void launch_gemm(const GemmArgs &g, bool ktail, hipStream_t st) {
    constexpr int R = B_KN ? gemm::kRingKn : gemm::kRingDefault;
    const dim3 grid(static_cast<unsigned>(g.tiles_per_xcd) * 8u), block(64 * gemm::waves_of(B_KN));
    if (ktail) hipLaunchKernelGGL((gemm::gemm_nt_kernel<MODE, true, SOFTCAP, false, B_KN, R>), grid, block, 0, st, g);
    else hipLaunchKernelGGL((gemm::gemm_nt_kernel<MODE, false, SOFTCAP, false, B_KN, R>), grid, block, 0, st, g);
}

// C (+)= A B^T over [M, N] with K split into `splits` ranges; the cross-entropy
// modes (OUT_STATS, OUT_GRAD) take their inputs from *ce and run unsplit.  With
// b_kn, B is stored k-major ([K][N], row stride ldb: C (+)= A B) and is read in
// place through transposing LDS reads (OUT_F32 only).
hipError_t gemm_nt(int mode, const void *A, int64_t lda, const void *B, int64_t ldb, void *C, int64_t ldc, int M,
                   int N, int K, int splits, int64_t c_split_stride, hipStream_t st,
                   const gemm::CeEpi *ce = nullptr, bool b_kn = false) {
    if (M <= 0 || N <= 0) return hipSuccess;
    if ((K & 7) || (lda & 7) || (ldb & 7) || (reinterpret_cast<uintptr_t>(A) & 15) ||
        (reinterpret_cast<uintptr_t>(B) & 15))
        return hipErrorInvalidValue;
    // 32-bit buffer offsets: a tile's rows plus one step of K read ahead (K-contiguous operands);
    // the whole [K][ldb] matrix (k-major B, whose N must be whole 16-byte chunks)
    const int64_t ldmax = b_kn ? lda : (lda > ldb ? lda : ldb);
    if (256 * ldmax * 2 + (static_cast<int64_t>(K) + 2 * gemm::BK) * 2 >= (int64_t(1) << 32)) return hipErrorInvalidValue;
    if (b_kn && ((N & 7) || static_cast<int64_t>(K) * ldb * 2 >= (int64_t(1) << 32) || mode != gemm::OUT_F32))
        return hipErrorInvalidValue;
    GemmArgs g;
    g.A = static_cast<const uint16_t *>(A);
    g.B = static_cast<const uint16_t *>(B);
    g.C = C;
    g.lda = lda;
    g.ldb = ldb;
    g.ldc = ldc;
    g.M = M;
    g.N = N;
    g.K = K;
    g.splits = splits;
    g.c_split_stride = c_split_stride;
    g.tiles_m = ceil_div(M, gemm::BM);
    g.tiles_n = ceil_div(N, gemm::BN);
    const int64_t total = static_cast<int64_t>(g.tiles_m) * g.tiles_n * splits;
    g.tiles_per_xcd = ceil_div(total, 8);
    g.ce = ce ? *ce : gemm::CeEpi{};
    const bool ktail = (K % gemm::BK) != 0;
    if (mode == gemm::OUT_STATS || mode == gemm::OUT_GRAD) {
        if (!ce || splits != 1) return hipErrorInvalidValue;
        const bool sc = ce->softcap > 0.0f;
        if (mode == gemm::OUT_STATS) {
            if (sc) launch_gemm<gemm::OUT_STATS, true>(g, ktail, st);
            else launch_gemm<gemm::OUT_STATS, false>(g, ktail, st);
        } else {
            if (sc) launch_gemm<gemm::OUT_GRAD, true>(g, ktail, st);
            else launch_gemm<gemm::OUT_GRAD, false>(g, ktail, st);
        }
    } else if (b_kn) launch_gemm<gemm::OUT_F32, false, true>(g, ktail, st);
    else if (mode == gemm::OUT_BF16) launch_gemm<gemm::OUT_BF16>(g, ktail, st);
    else if (mode == gemm::OUT_F32) launch_gemm<gemm::OUT_F32>(g, ktail, st);
    else launch_gemm<gemm::OUT_F32_ACC>(g, ktail, st);
    return hipGetLastError();
}

// K splits for a GEMM of `tiles` output tiles: the count (at most kFlceMaxSplitK,
// each split at least 8 K steps) whose workgroups fill the most of whole rounds
// over the compute units; ties go to fewer splits.
int choose_splits(int64_t tiles, int64_t K) {
    const int64_t cus = device_cu_count();
    const int64_t steps = (K + gemm::BK - 1) / gemm::BK;
    int best = 1;
    double best_eff = 0.0;
    for (int s = 1; s <= kFlceMaxSplitK && steps / s >= 8; ++s) {
        const int64_t wg = tiles * s;
        const double eff = static_cast<double>(wg) / static_cast<double>(((wg + cus - 1) / cus) * cus);
        if (eff > best_eff + 1e-9) {
            best_eff = eff;
            best = s;
        }
    }
    return best;
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }
int64_t round8(int64_t x) { return (x + 7) & ~static_cast<int64_t>(7); }
int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

}  // namespace

hipError_t launch_loss_fold(const float *loss_tok, int64_t n, const int64_t *counts, int reduction, float *loss_out,
                            hipStream_t st) {
    hipLaunchKernelGGL(loss_fold_kernel, dim3(1), dim3(1024), 0, st, loss_tok, n, counts, reduction, loss_out);
    return hipGetLastError();
}

int64_t flce_default_group_chunks(int64_t n, int64_t H, int64_t V, int64_t chunk) {
    const int64_t C = chunk < n ? chunk : (n > 0 ? n : 1);
    const int64_t nchunks = n > 0 ? (n + C - 1) / C : 1;
    const int64_t per_chunk = round_up(C, 64) * (V + H) * 2;
    const int64_t cpg = static_cast<int64_t>(kFlceGroupBytes) / per_chunk;
    return cpg < 1 ? 1 : (cpg > nchunks ? nchunks : cpg);
}

FlceLayout flce_layout(int64_t n, int64_t H, int64_t V, int64_t chunk, int64_t group_chunks, bool with_wt) {
    FlceLayout L;
    const int64_t C = chunk < n ? chunk : (n > 0 ? n : 1);
    L.chunk = C;
    const int64_t nchunks = n > 0 ? (n + C - 1) / C : 1;
    const int64_t cpg = group_chunks < 1 ? 1 : (group_chunks > nchunks ? nchunks : group_chunks);
    L.group = cpg * C;
    L.ldg = round_up(L.group, 64);
    size_t off = 0;
    L.off_wt = off;
    if (with_wt) off += align256(static_cast<size_t>(H) * V * 2);
    L.off_z = off;     off += align256(static_cast<size_t>(C) * V * 2);
    L.off_gt = off;    off += align256(static_cast<size_t>(V) * L.ldg * 2);
    L.off_ht = off;    off += align256(static_cast<size_t>(H) * L.ldg * 2);
    L.off_part = off;  off += align256(static_cast<size_t>(kFlceMaxSplitK) * C * H * 4);
    L.off_ce = off;    off += align256(ce_workspace_bytes(C));
    L.bytes = off;
    return L;
}

bool flce_plan(int64_t n, int64_t H, int64_t V, int64_t chunk, size_t bytes, int64_t *group_chunks, bool *with_wt) {
    int64_t group = flce_default_group_chunks(n, H, V, chunk);
    while (group > 1 && flce_layout(n, H, V, chunk, group, false).bytes > bytes) --group;
    *group_chunks = group;
    *with_wt = flce_layout(n, H, V, chunk, group, true).bytes <= bytes;
    return flce_layout(n, H, V, chunk, group, false).bytes <= bytes;
}

// The caller's optional second stream for the bandwidth-bound transposes, which
// then run beside the MFMA-bound GEMMs on the caller's stream: W^T beside the
// first chunk's logits GEMM, each G_c^T beside its grad_hidden GEMM.  Three
// events, created by the call and destroyed when it has enqueued everything,
// fork it from and join it back to the caller's stream, so a captured call
// captures both and nothing is kept between calls.  A second stream that is
// being captured while the caller's stream is not (or into another graph) is
// left alone: everything then runs on the caller's stream.
struct Aux {
    hipStream_t s = nullptr;   // null: no second stream
    hipEvent_t fork = nullptr, wt = nullptr, gt = nullptr;
    Aux() = default;
    Aux(const Aux &) = delete;
    Aux &operator=(const Aux &) = delete;
    ~Aux() {
        for (hipEvent_t e : {fork, wt, gt})
            if (e) (void)hipEventDestroy(e);   // released once the recorded work has run
    }
};

hipError_t aux_open(hipStream_t st, hipStream_t aux, Aux *A) {
    if (!aux || aux == st) return hipSuccess;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone, ca = hipStreamCaptureStatusNone;
    unsigned long long ids = 0, ida = 0;
    hipError_t e;
    if ((e = hipStreamGetCaptureInfo(st, &cs, &ids)) != hipSuccess) return e;
    if ((e = hipStreamGetCaptureInfo(aux, &ca, &ida)) != hipSuccess) return e;
    if (ca == hipStreamCaptureStatusActive && (cs != hipStreamCaptureStatusActive || ida != ids)) return hipSuccess;
    if ((e = hipEventCreateWithFlags(&A->fork, hipEventDisableTiming)) != hipSuccess ||
        (e = hipEventCreateWithFlags(&A->wt, hipEventDisableTiming)) != hipSuccess ||
        (e = hipEventCreateWithFlags(&A->gt, hipEventDisableTiming)) != hipSuccess)
        return e;
    A->s = aux;
    return hipSuccess;
}

// the second stream starts after everything enqueued on st so far
hipError_t fork_to(const Aux &A, hipStream_t st) {
    hipError_t e = hipEventRecord(A.fork, st);
    return e != hipSuccess ? e : hipStreamWaitEvent(A.s, A.fork, 0);
}

hipError_t launch_flce(const FlceArgs &f, hipStream_t st) {
    hipError_t e;
    const FlceLayout L = flce_layout(f.n, f.H, f.V, f.chunk, f.group_chunks, f.with_wt);
    char *ws = static_cast<char *>(f.workspace);
    uint16_t *z = reinterpret_cast<uint16_t *>(ws + L.off_z);
    uint16_t *gt = reinterpret_cast<uint16_t *>(ws + L.off_gt);
    uint16_t *ht = reinterpret_cast<uint16_t *>(ws + L.off_ht);
    float *part = reinterpret_cast<float *>(ws + L.off_part);
    void *ce_ws = ws + L.off_ce;
    const int64_t C = L.chunk, H = f.H, V = f.V;

    const bool resident = f.lse != nullptr;
    // counts (and a zeroed completion counter for the chunk CE calls); the
    // resident backward takes them from its stats pass
    if (!resident && (e = launch_ce_count(f.labels, f.n, V, f.ignore_index, f.counts, static_cast<unsigned long long *>(ce_ws),
                                          f.loss_out, st)) != hipSuccess)
        return e;
    if (f.n == 0) {
        const int64_t tot = V * H;
        hipLaunchKernelGGL(fill_zero_f32_kernel, dim3(2048), dim3(256), 0, st, f.grad_weight, tot);
        return hipGetLastError();
    }
    Aux A;
    if ((e = aux_open(st, f.aux, &A)) != hipSuccess) return e;
    const bool two = A.s != nullptr;
    // where the transposes of W and G_c go
    const hipStream_t ts = two ? A.s : st;
    uint16_t *wt = reinterpret_cast<uint16_t *>(ws + L.off_wt);
    bool wt_pending = false, gt_pending = false;
    if (f.with_wt) {   // W^T [H, V], on the second stream
        if ((two && (e = fork_to(A, st)) != hipSuccess) ||
            (e = transpose(f.weight, H, wt, V, static_cast<int>(V), static_cast<int>(V), static_cast<int>(H), ts)) !=
                hipSuccess ||
            (two && (e = hipEventRecord(A.wt, A.s)) != hipSuccess))
            return e;
        wt_pending = two;
    }
    const int tiles_dh = static_cast<int>(((C + gemm::BM - 1) / gemm::BM) * ((H + gemm::BN - 1) / gemm::BN));
    const int splits = choose_splits(tiles_dh, V);

    for (int64_t g0 = 0; g0 < f.n; g0 += L.group) {
        const int64_t gn = f.n - g0 < L.group ? f.n - g0 : L.group;
        for (int64_t c0 = g0; c0 < g0 + gn; c0 += C) {
            const int cn = static_cast<int>(g0 + gn - c0 < C ? g0 + gn - c0 : C);
            const bool last_in_group = c0 + cn >= g0 + gn;
            // the group's K ends on a whole 8-element chunk: pad the last chunk with zeros
            const int cpad = static_cast<int>(last_in_group ? round8(c0 + cn - g0) - (c0 - g0) : cn);
            const uint16_t *hc = static_cast<const uint16_t *>(f.hidden) + c0 * H;
            // H_c^T into columns [c0 - g0, ...) of the group's [H, ldg] buffer
            if ((e = transpose(hc, H, ht + (c0 - g0), L.ldg, cn, cpad, static_cast<int>(H), st)) != hipSuccess)
                return e;
            // the previous chunk's G^T transpose still reads z
            if (gt_pending && (e = hipStreamWaitEvent(st, A.gt, 0)) != hipSuccess) return e;
            gt_pending = false;
            if (resident) {
                // G_c straight from the GEMM's epilogue: Z_c stays in registers
                gemm::CeEpi ce{};
                ce.labels = f.labels + c0;
                ce.ignore_index = f.ignore_index;
                ce.softcap = f.softcap;
                ce.eps = f.eps;
                ce.lse = f.lse + c0;
                ce.q = f.q + c0;
                ce.grad_out = (f.reduction == 0 && f.grad_out) ? f.grad_out + c0 : f.grad_out;
                ce.counts = f.counts;
                ce.reduction = f.reduction;
                if ((e = gemm_nt(gemm::OUT_GRAD, hc, H, f.weight, H, z, V, cn, static_cast<int>(V),
                                 static_cast<int>(H), 1, 0, st, &ce)) != hipSuccess)
                    return e;
            } else {
                // Z_c = H_c W^T  -> bf16 [cn, V]
                if ((e = gemm_nt(gemm::OUT_BF16, hc, H, f.weight, H, z, V, cn, static_cast<int>(V), static_cast<int>(H),
                                 1, 0, st)) != hipSuccess)
                    return e;
                // G_c = CE(Z_c) in place, mean scale over all n tokens
                CEArgs a;
                a.logits = z;
                a.ld = V;
                a.n = cn;
                a.V = V;
                a.labels = f.labels + c0;
                a.count_labels = f.labels;
                a.count_n = f.n;
                a.ignore_index = f.ignore_index;
                a.eps = f.eps;
                a.softcap = f.softcap;
                a.reduction = f.reduction;
                a.grad_out = (f.reduction == 0 && f.grad_out) ? f.grad_out + c0 : f.grad_out;
                a.loss_tok = f.loss_tok + c0;
                a.loss_out = nullptr;
                a.argmax_out = nullptr;
                a.counts = f.counts;
                a.workspace = ce_ws;
                if ((e = launch_ce_fwd_bwd(a, true, st)) != hipSuccess) return e;
            }
            // G_c^T into columns [c0 - g0, ...) of the group's [V, ldg] buffer, on the second stream
            if ((two && (e = fork_to(A, st)) != hipSuccess) ||
                (e = transpose(z, V, gt + (c0 - g0), L.ldg, cn, cpad, static_cast<int>(V), ts)) != hipSuccess ||
                (two && (e = hipEventRecord(A.gt, A.s)) != hipSuccess))
                return e;
            gt_pending = two;
            if (wt_pending && (e = hipStreamWaitEvent(st, A.wt, 0)) != hipSuccess) return e;
            wt_pending = false;
            // dH_c = G_c W: split-K partials [splits, cn, H] fp32, folded to bf16
            // (W^T K-contiguous when the workspace holds it, else W itself, k-major)
            if ((e = f.with_wt ? gemm_nt(gemm::OUT_F32, z, V, wt, V, part, H, cn, static_cast<int>(H),
                                         static_cast<int>(V), splits, C * H, st)
                               : gemm_nt(gemm::OUT_F32, z, V, f.weight, H, part, H, cn, static_cast<int>(H),
                                         static_cast<int>(V), splits, C * H, st, nullptr, /*b_kn=*/true)) !=
                hipSuccess)
                return e;
            {
                const int64_t quads = static_cast<int64_t>(cn) * H / 4;
                const unsigned blocks = static_cast<unsigned>(std::min<int64_t>((quads + 255) / 256, 8192));
                hipLaunchKernelGGL(splitk_fold_kernel, dim3(blocks), dim3(256), 0, st, part, C * H, splits,
                                   static_cast<uint16_t *>(f.grad_hidden) + c0 * H, H, cn, static_cast<int>(H));
            }
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
        // the group's G^T is complete (this also joins the second stream back to st)
        if (gt_pending && (e = hipStreamWaitEvent(st, A.gt, 0)) != hipSuccess) return e;
        gt_pending = false;
        // dW (+)= G_g^T H_g over the group's tokens (K padded to a whole 8-element chunk)
        if ((e = gemm_nt(g0 == 0 ? gemm::OUT_F32 : gemm::OUT_F32_ACC, gt, L.ldg, ht, L.ldg, f.grad_weight, H,
                         static_cast<int>(V), static_cast<int>(H), static_cast<int>(round8(gn)), 1, 0, st)) !=
            hipSuccess)
            return e;
    }
    if (!resident && f.loss_out) return launch_loss_fold(f.loss_tok, f.n, f.counts, f.reduction, f.loss_out, st);
    return hipSuccess;
}

size_t flce_stats_bytes(int64_t n, int64_t V) {
    return static_cast<size_t>(n) * static_cast<size_t>(ceil_div(V, gemm::BN)) * kStatsFloats * sizeof(float);
}

hipError_t launch_flce_forward(const FlceFwdArgs &f, hipStream_t st) {
    hipError_t e;
    const int64_t tiles_n = ceil_div(f.V, gemm::BN);
    float *rec = static_cast<float *>(f.workspace);   // [n][tiles_n] records
    if (f.n > 0) {
        gemm::CeEpi ce{};
        ce.labels = f.labels;
        ce.ignore_index = f.ignore_index;
        ce.softcap = f.softcap;
        ce.eps = f.eps;
        ce.stats = rec;
        ce.rec_row_stride = tiles_n;
        ce.rec_tile_stride = 1;
        if ((e = gemm_nt(gemm::OUT_STATS, f.hidden, f.H, f.weight, f.H, nullptr, 0, static_cast<int>(f.n),
                         static_cast<int>(f.V), static_cast<int>(f.H), 1, 0, st, &ce)) != hipSuccess)
            return e;
    }
    return launch_ce_combine(rec, tiles_n, 1, tiles_n, f.labels, f.n, f.V, f.ignore_index, f.eps, f.reduction, f.lse,
                             f.q, f.loss_tok, f.loss_out, f.logp, f.ent, f.argmax_out, f.counts, st);
}

}  // namespace lce
