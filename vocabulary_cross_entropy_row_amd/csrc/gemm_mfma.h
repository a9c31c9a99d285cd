// bf16 MFMA GEMM for gfx950:  C[M, N] (+)= A[M, K] * B[N, K]^T
// A and B are bf16 with K contiguous (row strides lda, ldb in elements);
// C is row-major fp32 or bf16 (ldc).  lda and ldb must be multiples of 8
// and A, B 16-byte aligned (rows are fetched as 16-byte chunks straight into
// LDS); K must be a multiple of 8.  Used by the fused linear cross-entropy
// (Liger-Kernel PR "Add Liger Kernel support for Muse Glimmer", Summary /
// Memory): logits Z = H W^T, dH = G W, dW = G^T H, all accumulated in fp32.
//
// Tiling: a 512-thread workgroup (8 waves, two per SIMD) computes a 256 x 256
// tile; wave w owns rows 64 (w / 2) .. +64 and columns 128 (w % 2) .. +128 =
// 2 x 4 v_mfma_f32_32x32x16_bf16 tiles (128 fp32 accumulators per lane), so a
// SIMD always has a second wave to issue MFMAs while one waits.  With a k-major
// B the workgroup has 1024 threads (16 waves, four per SIMD) of 64 x 64 = 2 x 2
// tiles.  K advances in steps of 64.  Each step's A and B tiles (32 KB each) are fetched by
// buffer->LDS loads into LDS slots: with two stages the loads of step s+1 are
// issued at the start of step s; with the five-slot ring the streamed operand
// (B) of step s+2 goes out at the start of step s as well, into the fifth slot,
// so it has two steps to arrive.  One barrier per step hands the slots over.
// Fragment reads for sub-step kk+1 are issued while the MFMAs of kk run.
//
// LDS tile layout: row r holds its eight 16-byte K-chunks at positions
// p = c ^ swz(r).  A load instruction of a wave fills 1 KB = 8 rows x 8
// positions (lane l -> row l / 8, position l % 8) and fetches the global chunk
// that belongs there, so global reads stay coalesced, while the fragment reads
// (32 consecutive rows at one chunk) spread over all banks.
//
// MFMA operand layout (v_mfma_f32_32x32x16_bf16, checked on the device):
// lane l supplies A[l % 32][(l / 32) * 8 + j] and B^T[(l / 32) * 8 + j][l % 32]
// (j = 0..7); result register r of lane l is C[(r / 4) * 8 + (l / 32) * 4 + r % 4][l % 32].
//
// Two epilogues treat C as logits and never store it (the tile-resident form of
// the fused linear cross-entropy; the Muse Glimmer page's Summary asks for the
// loss without the [tokens, V] logits):
//   OUT_STATS  reduces each row of the fp32 tile to one stats record (running
//              max, sums of e^{z-m} and of e^{z-m} z without the target,
//              sum of z, first argmax of the raw logits, the target's z);
//   OUT_GRAD   recomputes the same tile and stores the bf16 gradient
//              s (p - (1 - eps)[j = y] - eps / V) dz/dx from the row's
//              log-sum-exp and 1 - p_y.
// Both passes run the identical main loop, so they see bitwise the same logits.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ce_device.h"

namespace lce {
namespace gemm {

#ifndef LCE_GEMM_BK
#define LCE_GEMM_BK 64
#endif
#ifndef LCE_GEMM_NSTAGE
#define LCE_GEMM_NSTAGE 2
#endif
#ifndef LCE_GEMM_NWAVES
#define LCE_GEMM_NWAVES 8
#endif
#ifndef LCE_GEMM_NWAVES_KN
#define LCE_GEMM_NWAVES_KN 16
#endif
#ifndef LCE_GEMM_RING
#define LCE_GEMM_RING 1
#endif
#ifndef LCE_GEMM_RING_KN
#define LCE_GEMM_RING_KN 0
#endif
constexpr int BM = 256, BN = 256, BK = LCE_GEMM_BK;
constexpr int NSTAGE = LCE_GEMM_NSTAGE;              // LDS stages; NSTAGE - 1 steps of loads in flight
constexpr int NWAVES = LCE_GEMM_NWAVES;              // waves of a K-contiguous GEMM's workgroup
constexpr int NWAVES_KN = LCE_GEMM_NWAVES_KN;        // ... and of one that reads B k-major
constexpr int waves_of(bool b_kn) { return b_kn ? NWAVES_KN : NWAVES; }
constexpr int WI = BM / 32 / (NWAVES / 2);           // A fragments (32 rows each) per wave, K-contiguous B
constexpr int WROWS = WI * 32;                       // tile rows per wave (two waves per row band)
constexpr int CPR = BK / 8;                          // 16-byte K chunks per tile row
constexpr int TILE_BYTES = BM * BK * 2;              // one operand tile of one stage
constexpr int STAGE_BYTES = 2 * TILE_BYTES;          // A | B
// The operand tiles live in LDS slots of TILE_BYTES.  Two stages (ring 0): four
// slots, both operands of step s+1 requested at the start of step s.  Ring 1 (B)
// or 2 (A): five slots, that operand requested two steps before it is used and
// the other one step before.
constexpr int kRingDefault = LCE_GEMM_RING;   // the ring of the K-contiguous GEMMs
constexpr int kRingKn = LCE_GEMM_RING_KN;      // ... and of the GEMM that reads B k-major
constexpr int nslots(int ring) { return ring ? 5 : 2 * NSTAGE; }
constexpr int lds_bytes(int ring) { return nslots(ring) * TILE_BYTES; }
constexpr int NBLK = TILE_BYTES / 1024;              // one-KB load blocks per operand tile
constexpr int KK = BK / 16;                          // MFMA K sub-steps per step
constexpr int kBufWord3 = 0x00020000;                // gfx9-family buffer descriptor word 3
static_assert(lds_bytes(0) <= 160 * 1024 && lds_bytes(1) <= 160 * 1024 && NBLK >= NWAVES_KN && (CPR == 4 || CPR == 8),
              "unsupported GEMM staging");
static_assert(kRingDefault == 0 || NSTAGE == 2, "the ring replaces the two stages");
static_assert((NWAVES == 8 || NWAVES == 4) && (NWAVES_KN == 16 || NWAVES_KN == 8), "wave counts");

enum OutMode { OUT_BF16 = 0, OUT_F32 = 1, OUT_F32_ACC = 2, OUT_STATS = 3, OUT_GRAD = 4 };

typedef __bf16 bf8 __attribute__((ext_vector_type(8)));
typedef float f16v __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void *lds_ptr;

// Inputs of the cross-entropy epilogues; GEMM row m is token m of the call.
struct CeEpi {
    const int64_t *labels;   // label of row m at labels[m]
    int64_t ignore_index;
    float softcap;           // > 0: z = T tanh(x / T); 0: z = x
    float eps;               // label smoothing (OUT_GRAD)
    float *stats;            // OUT_STATS: record of row m, column tile t at
    int64_t rec_row_stride;  //   stats + (m * rec_row_stride + t * rec_tile_stride) * 8
    int64_t rec_tile_stride;
    const float *lse;        // OUT_GRAD: log-sum-exp of row m at lse[m]
    const float *q;          // OUT_GRAD: 1 - p_y of row m at q[m]
    const float *grad_out;   // OUT_GRAD: NULL = 1; reduction none: grad_out[m]; else grad_out[0]
    const int64_t *counts;   // OUT_GRAD: counts[0] = valid labels, the mean's denominator
    int reduction;           // 0 none, 1 mean, 2 sum
};

struct GemmArgs {
    const uint16_t *A;   // [M, K] bf16, row stride lda
    const uint16_t *B;   // [N, K] bf16, row stride ldb
    void *C;             // [M, N] fp32 / bf16, row stride ldc (+ split * c_split_stride elements)
    int64_t lda, ldb, ldc;
    int M, N, K;
    int splits;          // K is divided into this many contiguous ranges of whole steps
    int64_t c_split_stride;
    int tiles_m, tiles_n;
    int tiles_per_xcd;   // ceil(total tiles / 8)
    CeEpi ce;            // OUT_STATS / OUT_GRAD only
};

// LDS position of K chunk c of row r is c ^ swz(r): the 16 rows that one LDS
// cycle serves for a fragment read (lanes 0-15, consecutive rows, one chunk)
// land on 16 distinct 16-byte bank groups of the 256-byte bank window.
__device__ __forceinline__ int swz(int r) { return (r / (16 / CPR)) & (CPR - 1); }

// k-major operand tiles ([k][256 columns], 512 bytes per k-row): the 16-byte chunk c of k-row kr sits
// at position c ^ kmswz(kr), so the four k-rows one transposing read touches fall in different bank
// windows.
__device__ __forceinline__ int kmswz(int kr) { return (kr & 3) << 2; }

// The MFMA operand fragment of columns cb .. cb + 31 for K sub-step kk from a k-major tile: lane l
// gets column cb + l % 32 at k = kk * 16 + (l / 32) * 8 + 0..7.  ds_read_b64_tr_b16 transposes
// 16-bit elements within each 16-lane group: result element j of lane d is element d % 4 of the
// 8 bytes that lane 4 j + d / 4 of the group addressed (checked on the device).  So source lane
// 4 j + q of group g addresses k-row kk * 16 + (g / 2) * 8 + t * 4 + j, columns
// cb + (g % 2) * 16 + 4 q .. + 3, and two reads (t = 0, 1) give the eight k values.
__device__ __forceinline__ bf8 km_frag(const unsigned char *tile, int kk, int cb, int lane) {
    typedef short v4s __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) v4s *lp4;
    const int g = lane >> 4, sl = lane & 15;
    const int col = cb + (g & 1) * 16 + (sl & 3) * 4;
    v4s h[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int kr = kk * 16 + (g >> 1) * 8 + t * 4 + (sl >> 2);
        const unsigned char *p = tile + kr * 512 + (((col >> 3) ^ kmswz(kr)) * 16) + (col & 7) * 2;
        h[t] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lp4)(p));
    }
    const v4s lo = h[0], hi = h[1];
    typedef short v8s __attribute__((ext_vector_type(8)));
    const v8s r = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    return __builtin_bit_cast(bf8, r);
}

// A buffer descriptor built from wave-uniform values, so it lives in SGPRs.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const void *p, uint32_t nrec) {
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32));
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>((static_cast<uint64_t>(hi) << 32) | lo), 0,
                                             __builtin_amdgcn_readfirstlane(nrec), kBufWord3);
}

// Epilogue layout: lane l of wave (wm, wn) holds tile column wn * 128 + j * 32 + l % 32
// of tile rows wm * 64 + i * 32 + (r / 4) * 8 + (l / 32) * 4 + r % 4.
__device__ __forceinline__ int epi_row(int wm, int i, int r, int lane) {
    return wm * WROWS + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
}

// Reductions over the 32 lanes of each half-wave (the lanes that share an accumulator row):
// four DPP steps leave every 16-lane row holding its row's result, then one swizzle exchanges
// rows 0 and 1 (2 and 3) of each half; every lane ends with its half's result.
constexpr int kSwzXor16 = 0x401F;   // ds_swizzle bit mode: lane ^ 16 within each 32
__device__ __forceinline__ float swz16_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), kSwzXor16));
}
__device__ __forceinline__ float half_max(float v) {
    v = fmaxf(v, dev::dpp_f<dev::kDppXor1>(v));
    v = fmaxf(v, dev::dpp_f<dev::kDppXor2>(v));
    v = fmaxf(v, dev::dpp_f<dev::kDppHalfMirror>(v));
    v = fmaxf(v, dev::dpp_f<dev::kDppMirror>(v));
    return fmaxf(v, swz16_f(v));
}
__device__ __forceinline__ float half_sum(float v) {
    v += dev::dpp_f<dev::kDppXor1>(v);
    v += dev::dpp_f<dev::kDppXor2>(v);
    v += dev::dpp_f<dev::kDppHalfMirror>(v);
    v += dev::dpp_f<dev::kDppMirror>(v);
    return v + swz16_f(v);
}
// (value, first index) of each half-wave, larger value first, then smaller index
__device__ __forceinline__ void half_argmax(float &v, int &i) {
    dev::argmax_step<dev::kDppXor1>(v, i);
    dev::argmax_step<dev::kDppXor2>(v, i);
    dev::argmax_step<dev::kDppHalfMirror>(v, i);
    dev::argmax_step<dev::kDppMirror>(v, i);
    dev::argmax_combine(v, i, swz16_f(v), __builtin_amdgcn_ds_swizzle(i, kSwzXor16));
}

// One stats record per row of the tile (columns [n0, n0 + 256) of the vocabulary).
template <bool SOFTCAP>
__device__ __forceinline__ void stats_epilogue(const GemmArgs &g, f16v (&acc)[WI][4], unsigned char *lds, int m0,
                                               int n0, int tn, int wm, int wn, int lane) {
    constexpr float kL2e = dev::kLog2e;
    int *sh_y = reinterpret_cast<int *>(lds);                 // [BM] target column in the tile, or -1
    float *sh_rec = reinterpret_cast<float *>(lds + BM * 4);  // [2 column halves][BM][8] partial records
    const int tid = threadIdx.x;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __syncthreads();   // every wave is done with the operand stages
    if (tid < BM) {
        int yr = -1;
        if (m0 + tid < g.M) {
            const int64_t y = g.ce.labels[m0 + tid];
            if (y != g.ce.ignore_index && y >= n0 && y < n0 + BN && y < g.N) yr = static_cast<int>(y - n0);
        }
        sh_y[tid] = yr;
    }
    __syncthreads();
    const dev::Cap cap{SOFTCAP ? 2.0f * kL2e / g.ce.softcap : 0.0f, g.ce.softcap};
    const int cbase = wn * 128 + (lane & 31);   // tile column of j = 0
    bool cv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) cv[j] = n0 + cbase + j * 32 < g.N;
    float *rec_w = sh_rec + wn * BM * 8;
#pragma unroll
    for (int i = 0; i < WI; ++i) {
#pragma unroll
        for (int rb = 0; rb < 16; rb += 8) {
            float lm[8], lx[8];
            int li[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                lm[u] = -FLT_MAX;
                lx[u] = -INFINITY;
                li[u] = 0x7fffffff;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if (!cv[j]) continue;
                    const float x = acc[i][j][rb + u];
                    const float z = SOFTCAP ? cap.z_of_r(cap.r_of(x)) : x;
                    acc[i][j][rb + u] = z;
                    lm[u] = fmaxf(lm[u], z);
                    if (x > lx[u]) {   // columns ascend with j: the first maximum stays
                        lx[u] = x;
                        li[u] = cbase + j * 32;
                    }
                }
            }
            // over the 32 lanes that share each row
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                lm[u] = half_max(lm[u]);
                half_argmax(lx[u], li[u]);
            }
            float sx[8], se[8], sz[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int rl = epi_row(wm, i, rb + u, lane);
                const int yr = sh_y[rl];
                const float mL = lm[u] * kL2e;
                sx[u] = 0.0f;
                se[u] = 0.0f;
                sz[u] = 0.0f;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if (!cv[j]) continue;
                    const float z = acc[i][j][rb + u];
                    float ex = dev::exp2_fast(fmaf(z, kL2e, -mL));
                    sz[u] += z;
                    if (cbase + j * 32 == yr) {   // the target: its z, and out of both sums
                        rec_w[rl * 8 + 6] = z;
                        rec_w[rl * 8 + 7] = 1.0f;
                        ex = 0.0f;
                    }
                    sx[u] += ex;
                    se[u] = fmaf(ex, z, se[u]);
                }
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                sx[u] = half_sum(sx[u]);
                se[u] = half_sum(se[u]);
                sz[u] = half_sum(sz[u]);
            }
            if ((lane & 31) == 0) {
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int rl = epi_row(wm, i, rb + u, lane);
                    float *o = rec_w + rl * 8;
                    o[0] = lm[u];
                    o[1] = sx[u];
                    o[2] = se[u];
                    o[3] = sz[u];
                    o[4] = lx[u];
                    o[5] = __int_as_float(li[u]);
                    const int yr = sh_y[rl] - wn * 128;
                    if (yr < 0 || yr >= 128) {   // no target in this half
                        o[6] = 0.0f;
                        o[7] = 0.0f;
                    }
                }
            }
        }
    }
    __syncthreads();
    // the two column halves of each row, in column order
    if (tid < BM && m0 + tid < g.M) {
        const float *a = sh_rec + tid * 8, *b = sh_rec + (BM + tid) * 8;
        const float M = fmaxf(a[0], b[0]);
        const float fa = dev::exp2_fast((a[0] - M) * kL2e), fb = dev::exp2_fast((b[0] - M) * kL2e);
        float amv = a[4];
        int am = __float_as_int(a[5]);
        if (b[4] > amv) {
            amv = b[4];
            am = __float_as_int(b[5]);
        }
        const bool ha = a[7] != 0.0f;
        float4 *o = reinterpret_cast<float4 *>(
            g.ce.stats + (static_cast<int64_t>(m0 + tid) * g.ce.rec_row_stride + tn * g.ce.rec_tile_stride) * 8);
        o[0] = make_float4(M, a[1] * fa + b[1] * fb, a[2] * fa + b[2] * fb, a[3] + b[3]);
        o[1] = make_float4(amv, __int_as_float(n0 + am), ha ? a[6] : b[6], ha ? 1.0f : b[7]);
    }
}

// The bf16 gradient of every element of the tile, stored at C[row, col].
template <bool SOFTCAP>
__device__ __forceinline__ void grad_epilogue(const GemmArgs &g, f16v (&acc)[WI][4], unsigned char *lds, int m0,
                                              int n0, int wm, int wn, int lane) {
    constexpr float kL2e = dev::kLog2e;
    float4 *sh_p = reinterpret_cast<float4 *>(lds);    // [BM] {lse log2e - log2|s|, |s| eps / V, target value, sign}
    int *sh_y = reinterpret_cast<int *>(lds + BM * 16);  // [BM] target column in the tile, or -1
    const int tid = threadIdx.x;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid < BM) {
        float4 p = make_float4(INFINITY, 0.0f, 0.0f, 1.0f);   // a zero scale: every element 0
        int yr = -1;
        const int m = m0 + tid;
        if (m < g.M) {
            const int64_t y = g.ce.labels[m];
            const bool valid = y != g.ce.ignore_index && y >= 0 && y < g.N;
            const float *go = g.ce.grad_out;
            const float gv = g.ce.reduction == 0 ? (go ? go[m] : 1.0f) : (go ? go[0] : 1.0f);
            const int64_t nv = g.ce.counts[0];
            const float scale =
                !valid ? 0.0f : (g.ce.reduction == 1 ? (nv > 0 ? gv / static_cast<float>(nv) : 0.0f) : gv);
            if (scale != 0.0f) {
                const float as = fabsf(scale);
                p.x = g.ce.lse[m] * kL2e - log2f(as);
                p.y = g.ce.eps / static_cast<float>(g.N) * as;
                p.z = as * (g.ce.eps - g.ce.q[m]) - p.y;   // p_y - 1 = -q, kept exact
                p.w = scale < 0.0f ? -1.0f : 1.0f;
                if (y >= n0 && y < n0 + BN) yr = static_cast<int>(y - n0);
            }
        }
        sh_p[tid] = p;
        sh_y[tid] = yr;
    }
    __syncthreads();
    const dev::Cap cap{SOFTCAP ? 2.0f * kL2e / g.ce.softcap : 0.0f, g.ce.softcap};
    const int cbase = wn * 128 + (lane & 31);
    __bf16 *C = static_cast<__bf16 *>(g.C);
#pragma unroll
    for (int i = 0; i < WI; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int rl = epi_row(wm, i, r, lane);
            if (m0 + rl >= g.M) continue;
            const float4 P = sh_p[rl];
            const int yr = sh_y[rl];
            __bf16 *crow = C + static_cast<int64_t>(m0 + rl) * g.ldc + n0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int c = cbase + j * 32;
                if (n0 + c >= g.N) continue;
                const float x = acc[i][j][r];
                float z = x, ch = P.w;
                if constexpr (SOFTCAP) {
                    float rr, qq;
                    cap.r_q(x, rr, qq);
                    z = cap.z_of_r(rr);
                    ch *= dev::Cap::chain(rr, qq);
                }
                const float pe = dev::exp2_fast(fmaf(z, kL2e, -P.x));
                const float gval = c == yr ? P.z : pe - P.y;
                crow[c] = static_cast<__bf16>(gval * ch);   // RNE
            }
        }
    }
}

// KTAIL: K is not a multiple of BK, so each load checks its K column; otherwise
// the K position rides in the scalar offset and the per-lane offsets are fixed.
template <int MODE, bool KTAIL, bool SOFTCAP = false, bool A_KM = false, bool B_KN = false, int RING = 0>
__global__ __launch_bounds__(64 * waves_of(B_KN)) __attribute__((amdgpu_waves_per_eu(waves_of(B_KN) / 4, waves_of(B_KN) / 4))) void gemm_nt_kernel(GemmArgs g) {
    constexpr int NSLOT = nslots(RING);
    constexpr int NW = waves_of(B_KN);                  // waves of this workgroup
    constexpr int LOADS = NBLK / NW;                    // 1 KB loads per wave per operand per step
    // Wave tile: WIK A fragments x WJ B fragments of 32 x 32.  With a k-major B (two transposing
    // LDS reads per fragment) the workgroup has four waves per SIMD of 2 x 2 fragments: measured
    // faster there, slower for the K-contiguous GEMMs.
    constexpr int WJ = B_KN ? 2 : 4;                    // B fragments per wave
    constexpr int WAVES_N = BN / (WJ * 32);             // waves across the tile's columns
    constexpr int WIK = BM / 32 / (NW / WAVES_N);       // A fragments per wave
    constexpr int WRK = WIK * 32;                       // tile rows per wave
    static_assert(NW % WAVES_N == 0 && WIK >= 1 && LOADS >= 1, "wave tiling");
    static_assert(!B_KN || (MODE != OUT_STATS && MODE != OUT_GRAD), "the epilogues take 64 x 128 wave tiles");
    __shared__ __attribute__((aligned(1024))) unsigned char lds[lds_bytes(RING)];

    // XCD-aware tile order: workgroups are dealt round-robin over the 8 XCDs;
    // each XCD walks a contiguous range of the logical tile order.  That order
    // takes row tiles in groups of GROUP_M and, within a group, walks the
    // column tiles with the group's row tiles fastest (then the K split), so
    // the ~32 tiles an XCD runs at once form a GROUP_M x 8 block sharing
    // GROUP_M + 8 operand panels in its L2.
    constexpr int GROUP_M = 4;
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int t = xcd * g.tiles_per_xcd + slot;
    const int total = g.tiles_m * g.tiles_n * g.splits;
    if (slot >= g.tiles_per_xcd || t >= total) return;
    const int mn = t % (g.tiles_m * g.tiles_n);
    const int first_m = (mn / (GROUP_M * g.tiles_n)) * GROUP_M;
    const int gm = min(GROUP_M, g.tiles_m - first_m);
    const int within = mn - first_m * g.tiles_n;
    const int tm = first_m + within % gm;
    const int tn = within / gm;
    const int ks = t / (g.tiles_m * g.tiles_n);
    const int m0 = tm * BM, n0 = tn * BN;
    const int ksteps_total = (g.K + BK - 1) / BK;
    const int kbeg = static_cast<int>((static_cast<int64_t>(ksteps_total) * ks) / g.splits);
    const int kend = static_cast<int>((static_cast<int64_t>(ksteps_total) * (ks + 1)) / g.splits);

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    // K-contiguous operands: the descriptors cover exactly the tile's valid rows, so rows past M or N
    // read as zeros.  k-major operands ([K][rows], A_KM / B_KN): the descriptor starts at the tile's
    // first column and covers rows k < K, so rows past K read as zeros; columns past M or N are masked
    // per lane.
    const int a_rows = min(BM, g.M - m0), b_rows = min(BN, g.N - n0);
    const __amdgpu_buffer_rsrc_t rsA =
        A_KM ? uniform_rsrc(g.A + m0, static_cast<uint32_t>(static_cast<int64_t>(g.K) * g.lda - m0) * 2u)
             : uniform_rsrc(g.A + static_cast<int64_t>(m0) * g.lda,
                            static_cast<uint32_t>(a_rows) * static_cast<uint32_t>(g.lda) * 2u);
    const __amdgpu_buffer_rsrc_t rsB =
        B_KN ? uniform_rsrc(g.B + n0, static_cast<uint32_t>(static_cast<int64_t>(g.K) * g.ldb - n0) * 2u)
             : uniform_rsrc(g.B + static_cast<int64_t>(n0) * g.ldb,
                            static_cast<uint32_t>(b_rows) * static_cast<uint32_t>(g.ldb) * 2u);

    // this wave's load blocks: byte offsets at k = 0 and their K columns (K-contiguous), or their
    // column validity (k-major: block b holds k-rows 2b, 2b+1 of 32 swizzled 16-byte chunks)
    // (arrays of a bound that does not depend on the template arguments: with a dependent
    // bound the host pass leaves some instantiations' launch stubs undefined)
    constexpr int kMaxLoads = NBLK / 4;
    static_assert(LOADS <= kMaxLoads, "load slots");
    uint32_t voffA[kMaxLoads], voffB[kMaxLoads];
    int kcol[kMaxLoads];
    bool okA[kMaxLoads], okB[kMaxLoads];
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
        const int r = (j * NW + wave) * (64 / CPR) + lane / CPR;
        const int c = (lane % CPR) ^ swz(r);
        kcol[j] = c * 8;
        voffA[j] = static_cast<uint32_t>(r) * static_cast<uint32_t>(g.lda) * 2u + c * 16u;
        voffB[j] = static_cast<uint32_t>(r) * static_cast<uint32_t>(g.ldb) * 2u + c * 16u;
        const int kr = 2 * (j * NW + wave) + (lane >> 5);
        const int kc = (lane & 31) ^ kmswz(kr);
        if constexpr (A_KM) {
            voffA[j] = (static_cast<uint32_t>(kr) * static_cast<uint32_t>(g.lda) + kc * 8u) * 2u;
            okA[j] = m0 + kc * 8 < g.M;
        }
        if constexpr (B_KN) {
            voffB[j] = (static_cast<uint32_t>(kr) * static_cast<uint32_t>(g.ldb) + kc * 8u) * 2u;
            okB[j] = n0 + kc * 8 < g.N;
        }
    }

    // load j of one operand of step `step` into operand slot `slot`
    auto issue = [&](int step, int slot, int j, bool isB) {
        unsigned char *dst = lds + slot * TILE_BYTES + (j * NW + wave) * 1024;
        const int k0 = step * BK;
        if ((isB && B_KN) || (!isB && A_KM)) {
            // k-major: the step's rows are k0 .. k0 + 63 (past K: outside the descriptor)
            uint32_t v = (isB ? voffB[j] : voffA[j]) +
                         static_cast<uint32_t>(k0) * static_cast<uint32_t>(isB ? g.ldb : g.lda) * 2u;
            if (!(isB ? okB[j] : okA[j])) v = 0xFFFFFFF0u;   // past M or N: out of range, reads zeros
            __builtin_amdgcn_raw_ptr_buffer_load_lds(isB ? rsB : rsA, (lds_ptr)dst, 16, v, 0, 0, 0);
        } else if constexpr (KTAIL) {
            uint32_t v = (isB ? voffB[j] : voffA[j]) + static_cast<uint32_t>(k0) * 2u;
            if (k0 + kcol[j] >= g.K) v = 0xFFFFFFF0u;   // past K: out of range, reads zeros
            __builtin_amdgcn_raw_ptr_buffer_load_lds(isB ? rsB : rsA, (lds_ptr)dst, 16, v, 0, 0, 0);
        } else {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(isB ? rsB : rsA, (lds_ptr)dst, 16, isB ? voffB[j] : voffA[j],
                                                     k0 * 2, 0, 0);
        }
    };
    auto read_frags = [&](int slot_a, int slot_b, int kk, bf8 *af, bf8 *bfr) {
        const unsigned char *At = lds + slot_a * TILE_BYTES;
        const unsigned char *Bt = lds + slot_b * TILE_BYTES;
        const int c = kk * 2 + (lane >> 5);
#pragma unroll
        for (int i = 0; i < WIK; ++i) {
            if constexpr (A_KM) {
                af[i] = km_frag(At, kk, wm * WRK + i * 32, lane);
            } else {
                const int r = wm * WRK + i * 32 + (lane & 31);
                af[i] = *reinterpret_cast<const bf8 *>(At + (r * CPR + (c ^ swz(r))) * 16);
            }
        }
#pragma unroll
        for (int j = 0; j < WJ; ++j) {
            if constexpr (B_KN) {
                bfr[j] = km_frag(Bt, kk, wn * WJ * 32 + j * 32, lane);
            } else {
                const int r = wn * WJ * 32 + j * 32 + (lane & 31);
                bfr[j] = *reinterpret_cast<const bf8 *>(Bt + (r * CPR + (c ^ swz(r))) * 16);
            }
        }
    };
    // wait until at most `steps` steps of this wave's loads are outstanding
    // (loads complete in issue order; the count must be an immediate)
    auto wait_steps = [&](int steps) {
        constexpr int L = 2 * LOADS;
        if (steps <= 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        else if (steps == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(L) : "memory");
        else if (steps == 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * L) : "memory");
        else asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * L) : "memory");
    };

    // Spread the fragment reads of the next sub-step (and in sub-step 0 the global loads) between this
    // sub-step's MFMAs: all reads go out in the first NM - 2 MFMA slots, two to a slot where there are
    // more reads than slots (the transposing reads of k-major operands), so the last ones have two
    // MFMAs to land before the next sub-step needs them.
    auto interleave = [&](int kk) {
        constexpr int NM = WIK * WJ;                                    // MFMAs per sub-step
        constexpr int NR = (A_KM ? 2 * WIK : WIK) + (B_KN ? 2 * WJ : WJ);   // LDS reads per sub-step
        constexpr int NS = NM - 2;
        static_assert(NR <= 4 * NS, "at most four reads per MFMA slot");
#pragma unroll
        for (int q = 0; q < NM; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                // MFMA
            const int nr = q < NS ? NR / NS + (q < NR % NS ? 1 : 0) : 0;
            if (nr == 4) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);                   // LDS reads
            else if (nr == 3) __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
            else if (nr == 2) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            else if (nr == 1) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            if (kk == 0 && q < 2 * LOADS) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read
        }
    };

    const int nsteps = kend - kbeg;
    f16v acc[WIK][WJ];
#pragma unroll
    for (int i = 0; i < WIK; ++i)
#pragma unroll
        for (int j = 0; j < WJ; ++j) acc[i][j] = (f16v){};
    bf8 af0[WIK], bf0[WJ], af1[WIK], bf1[WJ];
    if constexpr (RING != 0) {
        // Operand tiles in request order: T(2s) is the early operand of step s (B for RING 1, A for 2),
        // T(2s+1) the other; T(i) lives in slot i mod 5.  At the start of step s the slots of step s-1
        // are free and take T(2s+3) (the late operand of step s+1) and T(2s+4) (the early operand of
        // step s+2): the early operand is requested two steps before it is used, the late one one step.
        constexpr bool EARLY_B = RING == 1;
        auto issue_tile = [&](int step, int slot, bool isB) {
#pragma unroll
            for (int j = 0; j < LOADS; ++j) issue(step, slot, j, isB);
        };
        auto wrap = [](int x) { return x >= NSLOT ? x - NSLOT : x; };
        if (nsteps > 0) {
            issue_tile(kbeg, 0, EARLY_B);
            issue_tile(kbeg, 1, !EARLY_B);
            if (nsteps > 1) {
                issue_tile(kbeg + 1, 2, EARLY_B);
                asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LOADS) : "memory");   // T(0), T(1)
            } else {
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            }
            asm volatile("s_barrier" ::: "memory");
            read_frags(EARLY_B ? 1 : 0, EARLY_B ? 0 : 1, 0, af0, bf0);
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);
        int base = 0;   // slot of T(2s)
        for (int s = 0; s < nsteps; ++s) {
            const int s1 = wrap(base + 1), s2 = wrap(base + 2), s3 = wrap(base + 3), s4 = wrap(base + 4);
            const int sa = EARLY_B ? s1 : base, sb = EARLY_B ? base : s1;        // this step's A and B
            const int na = EARLY_B ? s3 : s2, nb = EARLY_B ? s2 : s3;            // step s+1's
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                bf8 *ac = (kk & 1) ? af1 : af0, *bc = (kk & 1) ? bf1 : bf0;
                bf8 *an = (kk & 1) ? af0 : af1, *bn = (kk & 1) ? bf0 : bf1;
                __builtin_amdgcn_sched_barrier(0);
                if (kk == 0) {
                    // s3 and s4 held step s-1's tiles, which every wave read before the barrier that ended it
                    if (s + 1 < nsteps) issue_tile(kbeg + s + 1, s3, !EARLY_B);
                    if (s + 2 < nsteps) issue_tile(kbeg + s + 2, s4, EARLY_B);
                }
                if (kk + 1 < KK) {
                    read_frags(sa, sb, kk + 1, an, bn);
                } else {
                    // step s+1's tiles have landed for this wave (only T(2s+4) may be outstanding);
                    // after the barrier, for every wave
                    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                    if (s + 2 < nsteps) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LOADS) : "memory");
                    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                    asm volatile("s_barrier" ::: "memory");
                    read_frags(na, nb, 0, an, bn);
                }
#pragma unroll
                for (int i = 0; i < WIK; ++i)
#pragma unroll
                    for (int j = 0; j < WJ; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ac[i], bc[j], acc[i][j], 0, 0, 0);
                interleave(kk);
            }
            base = s2;
        }
    } else {
        constexpr int D = NSTAGE - 1;   // steps of loads in flight ahead of the one being consumed
        static_assert(D >= 1 && D <= 4, "wait_steps covers up to three outstanding steps");
        if (nsteps > 0) {
            for (int p = 0; p < D && p < nsteps; ++p) {
#pragma unroll
                for (int j = 0; j < LOADS; ++j) {
                    issue(kbeg + p, 2 * p, j, false);
                    issue(kbeg + p, 2 * p + 1, j, true);
                }
            }
            wait_steps(min(D, nsteps) - 1);                // this wave's loads of the first step
            asm volatile("s_barrier" ::: "memory");       // ... and every wave's
            read_frags(0, 1, 0, af0, bf0);
        }
        // settle the scalar loads so the LDS waits inside the loop count precisely
        // (s_waitcnt lgkmcnt(0), vmcnt and expcnt left open)
        __builtin_amdgcn_s_waitcnt(0xC07F);

        int st = 0;   // stage of step s
        for (int s = 0; s < nsteps; ++s) {
            const int st_next = st + 1 == NSTAGE ? 0 : st + 1;
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                bf8 *ac = (kk & 1) ? af1 : af0, *bc = (kk & 1) ? bf1 : bf0;
                bf8 *an = (kk & 1) ? af0 : af1, *bn = (kk & 1) ? bf0 : bf1;
                __builtin_amdgcn_sched_barrier(0);
                if (kk == 0 && s + D < nsteps) {
                    // the stage of step s+D was last read in step s-1, which every wave
                    // finished before the barrier that ended it
                    const int st_issue = st == 0 ? NSTAGE - 1 : st - 1;
#pragma unroll
                    for (int j = 0; j < LOADS; ++j) {
                        issue(kbeg + s + D, 2 * st_issue, j, false);
                        issue(kbeg + s + D, 2 * st_issue + 1, j, true);
                    }
                }
                if (kk + 1 < KK) {
                    read_frags(2 * st, 2 * st + 1, kk + 1, an, bn);
                } else {
                    // this wave's fragments of stage st are in registers and its loads
                    // of step s+1 have landed; after the barrier so are everyone's
                    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                    wait_steps(min(s + D, nsteps - 1) - (s + 1));
                    asm volatile("s_barrier" ::: "memory");
                    read_frags(2 * st_next, 2 * st_next + 1, 0, an, bn);
                }
#pragma unroll
                for (int i = 0; i < WIK; ++i)
#pragma unroll
                    for (int j = 0; j < WJ; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ac[i], bc[j], acc[i][j], 0, 0, 0);
                interleave(kk);
            }
            st = st_next;
        }
    }

    if constexpr (MODE == OUT_STATS) {
        stats_epilogue<SOFTCAP>(g, acc, lds, m0, n0, tn, wm, wn, lane);
        return;
    } else if constexpr (MODE == OUT_GRAD) {
        grad_epilogue<SOFTCAP>(g, acc, lds, m0, n0, wm, wn, lane);
        return;
    }
    // epilogue: lane holds column n0 + wn*32 WJ + j*32 + lane%32 of rows
    // m0 + wm*32 WIK + i*32 + (r/4)*8 + (lane/32)*4 + r%4
    const int col_base = n0 + wn * WJ * 32 + (lane & 31);
    const int row_base = m0 + wm * WRK + (lane >> 5) * 4;
#pragma unroll
    for (int i = 0; i < WIK; ++i) {
#pragma unroll
        for (int jh = 0; jh < WJ / 2; ++jh) {
            float old[2][16];
            if constexpr (MODE == OUT_F32_ACC) {
                // all loads of this group are issued before any of its stores
#pragma unroll
                for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int row = row_base + i * 32 + (r >> 2) * 8 + (r & 3);
                        const int col = col_base + (jh * 2 + jj) * 32;
                        old[jj][r] = (row < g.M && col < g.N)
                                         ? static_cast<const float *>(g.C)[static_cast<int64_t>(row) * g.ldc + col]
                                         : 0.0f;
                    }
            }
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                const int j = jh * 2 + jj;
                const int col = col_base + j * 32;
                if (col >= g.N) continue;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = row_base + i * 32 + (r >> 2) * 8 + (r & 3);
                    if (row >= g.M) continue;
                    const int64_t off =
                        static_cast<int64_t>(row) * g.ldc + col + static_cast<int64_t>(ks) * g.c_split_stride;
                    const float v = acc[i][j][r];
                    if constexpr (MODE == OUT_BF16) {
                        static_cast<__bf16 *>(g.C)[off] = static_cast<__bf16>(v);   // RNE
                    } else if constexpr (MODE == OUT_F32) {
                        static_cast<float *>(g.C)[off] = v;
                    } else {
                        static_cast<float *>(g.C)[off] = old[jj][r] + v;
                    }
                }
            }
        }
    }
}

}  // namespace gemm
}  // namespace lce
