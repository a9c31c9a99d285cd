// bf16 MFMA GEMM for gfx950:  C[M, N] (+)= A[M, K] * B[N, K]^T
// A and B are bf16 with K contiguous (row strides lda, ldb in elements);
// C is row-major fp32 or bf16 (ldc).  K, lda and ldb must be multiples of 8
// (whole 16-byte chunks: the K tail is skipped chunk by chunk, and rows must
// be 16-byte aligned for the direct-to-LDS loads).  Used by the fused linear
// cross-entropy (Liger-Kernel PR "Add Liger Kernel support for Muse
// Glimmer", Summary / Memory): logits Z = H W^T, dH = G W, dW += G^T H, with
// fp32 accumulation.
//
// Tiling: a 256-thread workgroup computes a 256 x 256 tile; its four waves
// own 128 x 128 quadrants = 4 x 4 v_mfma_f32_32x32x16_bf16 tiles each
// (256 fp32 accumulators per lane).  K advances in steps of 64.  Each step's
// A and B tiles (32 KB each) are staged in LDS by direct buffer->LDS loads
// into two alternating buffers, so the loads of step t+1 overlap the MFMAs
// of step t.
//
// LDS tile layout: row r of a tile holds its eight 16-byte K-chunks at
// positions p = c ^ swz(r), swz(r) = (r >> 1) & 7.  A load instruction of a
// wave fills 1 KB = 8 rows x 8 positions contiguously (lane l -> row l / 8,
// position l % 8) and each lane fetches the global chunk that belongs at its
// position, so global reads stay coalesced (a row's 128 bytes per 8 lanes)
// while the MFMA fragment reads (32 rows, one chunk each) hit 16 distinct
// bank groups per 16 lanes.
//
// MFMA operand layout (v_mfma_f32_32x32x16_bf16, verified on the device):
// lane l supplies A[l % 32][(l / 32) * 8 + j] and B^T[(l / 32) * 8 + j][l % 32]
// (j = 0..7); result register r of lane l is C[(r / 4) * 8 + (l / 32) * 4 + r % 4][l % 32].
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lce {
namespace gemm {

constexpr int BM = 256, BN = 256, BK = 64, NTHR = 256;
constexpr int TILE_BYTES = BM * BK * 2;            // one operand tile: 32 KB
constexpr int kBufWord3 = 0x00020000;              // gfx9-family buffer descriptor word 3

enum OutMode { OUT_BF16 = 0, OUT_F32 = 1, OUT_F32_ACC = 2 };

typedef __bf16 bf8 __attribute__((ext_vector_type(8)));
typedef float f16v __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct GemmArgs {
    const uint16_t *A;   // [M, K] bf16, row stride lda
    const uint16_t *B;   // [N, K] bf16, row stride ldb
    void *C;             // [M, N] fp32 / bf16, row stride ldc (+ split * c_split_stride elements)
    int64_t lda, ldb, ldc;
    int M, N, K;
    int splits;          // K is divided into this many contiguous ranges (multiples of BK)
    int64_t c_split_stride;
    int tiles_m, tiles_n;
    int tiles_per_xcd;   // ceil(total tiles / 8)
};

__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

// Issue this wave's share (8 of 32 one-KB blocks) of one operand tile: rows
// [row0, row0 + 256) of a K-contiguous matrix, K columns [k0, k0 + 64).
__device__ __forceinline__ void stage_tile(const uint16_t *mat, int64_t ld, int rows_valid, int k0, int K,
                                           unsigned char *lds_tile, int wave, int lane) {
    // the descriptor covers exactly the tile's valid rows: rows past the
    // matrix read as zeros
    const uint32_t nrec = static_cast<uint32_t>(rows_valid > 0 ? rows_valid : 0) * static_cast<uint32_t>(ld) * 2u;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(mat), 0, nrec, kBufWord3);
    const int p = lane & 7;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int blk = j * 4 + wave;           // 0..31: rows [8 blk, 8 blk + 8)
        const int r = blk * 8 + (lane >> 3);
        const int c = p ^ swz(r);               // the global chunk stored at position p
        const int kk = k0 + c * 8;
        uint32_t voff = static_cast<uint32_t>(r) * static_cast<uint32_t>(ld) * 2u + static_cast<uint32_t>(kk) * 2u;
        if (kk >= K) voff = 0xFFFFFFF0u;        // past K: out of range, reads zeros
        typedef __attribute__((address_space(3))) void *lptr;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lptr)(lds_tile + blk * 1024), 16, voff, 0, 0, 0);
    }
}

__device__ __forceinline__ void wait_vmcnt_le16() { asm volatile("s_waitcnt vmcnt(16)" ::: "memory"); }
__device__ __forceinline__ void wait_vmcnt_0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

template <int MODE>
__global__ __launch_bounds__(NTHR) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_nt_kernel(GemmArgs g) {
    __shared__ __attribute__((aligned(1024))) unsigned char lds[2 * 2 * TILE_BYTES];   // [stage][A|B]

    // XCD-aware tile order: workgroups are dealt round-robin over the 8 XCDs;
    // each XCD walks a contiguous range of the logical tile order, so tiles
    // that share an operand tile run close together on the same L2.
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int t = xcd * g.tiles_per_xcd + slot;
    const int total = g.tiles_m * g.tiles_n * g.splits;
    if (slot >= g.tiles_per_xcd || t >= total) return;
    // logical order: split-major, then n, then m (consecutive tiles share B)
    const int tm = t % g.tiles_m;
    const int tn = (t / g.tiles_m) % g.tiles_n;
    const int ks = t / (g.tiles_m * g.tiles_n);
    const int m0 = tm * BM, n0 = tn * BN;

    const int ksteps_total = (g.K + BK - 1) / BK;
    const int kbeg = static_cast<int>((static_cast<int64_t>(ksteps_total) * ks) / g.splits);
    const int kend = static_cast<int>((static_cast<int64_t>(ksteps_total) * (ks + 1)) / g.splits);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const uint16_t *Ab = g.A + static_cast<int64_t>(m0) * g.lda;
    const uint16_t *Bb = g.B + static_cast<int64_t>(n0) * g.ldb;
    const int a_rows = min(BM, g.M - m0), b_rows = min(BN, g.N - n0);

    f16v acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = (f16v){};

    auto stage = [&](int step, int buf) {
        unsigned char *base = lds + buf * 2 * TILE_BYTES;
        stage_tile(Ab, g.lda, a_rows, step * BK, g.K, base, wave, lane);
        stage_tile(Bb, g.ldb, b_rows, step * BK, g.K, base + TILE_BYTES, wave, lane);
    };

    if (kbeg < kend) stage(kbeg, 0);
    for (int s = kbeg; s < kend; ++s) {
        const int buf = (s - kbeg) & 1;
        if (s + 1 < kend) {
            stage(s + 1, buf ^ 1);
            wait_vmcnt_le16();   // this wave's 16 loads of step s have landed
        } else {
            wait_vmcnt_0();
        }
        __syncthreads();         // ... and every other wave's
        const unsigned char *At = lds + buf * 2 * TILE_BYTES;
        const unsigned char *Bt = At + TILE_BYTES;
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            const int c = kk * 2 + (lane >> 5);
            bf8 af[4], bfr[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = wm * 128 + i * 32 + (lane & 31);
                af[i] = *reinterpret_cast<const bf8 *>(At + (r * 8 + (c ^ swz(r))) * 16);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = wn * 128 + j * 32 + (lane & 31);
                bfr[j] = *reinterpret_cast<const bf8 *>(Bt + (r * 8 + (c ^ swz(r))) * 16);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
        __syncthreads();         // done reading this buffer before it is refilled
    }

    // epilogue: lane holds column n0 + wn*128 + j*32 + lane%32 of rows
    // m0 + wm*128 + i*32 + (r/4)*8 + (lane/32)*4 + r%4
    const int col_base = n0 + wn * 128 + (lane & 31);
    const int row_base = m0 + wm * 128 + (lane >> 5) * 4;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int col = col_base + j * 32;
            if (col >= g.N) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = row_base + i * 32 + (r >> 2) * 8 + (r & 3);
                if (row >= g.M) continue;
                const int64_t off = static_cast<int64_t>(row) * g.ldc + col + static_cast<int64_t>(ks) * g.c_split_stride;
                const float v = acc[i][j][r];
                if constexpr (MODE == OUT_BF16) {
                    static_cast<__bf16 *>(g.C)[off] = static_cast<__bf16>(v);   // RNE
                } else if constexpr (MODE == OUT_F32) {
                    static_cast<float *>(g.C)[off] = v;
                } else {
                    static_cast<float *>(g.C)[off] += v;
                }
            }
        }
}

}  // namespace gemm
}  // namespace lce
