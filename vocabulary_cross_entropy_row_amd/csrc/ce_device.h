// Device helpers shared by the cross-entropy kernels (gfx950, wave64).
#pragma once

#include <float.h>
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "lce_internal.h"

namespace lce {
namespace dev {

// 16-byte vector as a clang vector type (usable with the non-temporal builtins).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int NT = kRowThreads;
constexpr int NWAVE = NT / 64;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float exp2_fast(float t) { return __builtin_amdgcn_exp2f(t); }
__device__ __forceinline__ float rcp_fast(float t) { return __builtin_amdgcn_rcpf(t); }

// Hide register-resident data from the optimiser at a pass boundary.  Without
// this the compiler keeps every widened (fp32) element of one pass alive for
// reuse in the next, doubling the row's register footprint and spilling.
template <int K>
__device__ __forceinline__ void opaque_regs(u32x4 (&v)[K]) {
#pragma unroll
    for (int k = 0; k < K; ++k) asm volatile("" : "+v"(v[k]));
}

// Wait for every outstanding vector-memory operation of this wave (including
// loads that write LDS directly, which the compiler does not track).
__device__ __forceinline__ void wait_vmem_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Softcap support.  With u = x / T:  tanh(u) = 1 - 2 r,  r = 1 / (1 + e^{2u}),
// so z = T - 2 T r and dz/dx = 1 - tanh^2(u) = 4 r (1 - r).  r comes from the
// hardware base-2 exponential and reciprocal.
struct Cap {
    float c2;   // 2 log2(e) / T
    float T;
    __device__ __forceinline__ float r_of(float x) const { return rcp_fast(1.0f + exp2_fast(x * c2)); }
    __device__ __forceinline__ float z_of_r(float r) const { return fmaf(-2.0f * T, r, T); }
    // r and q = 1 - r for the chain factor.  q is formed as r e (e = e^{2u}), not
    // as 1 - r: where tanh saturates below zero r rounds towards 1 and 1 - r would
    // lose all its digits, while r e keeps full relative precision.  Where tanh
    // saturates above zero e overflows to inf and r to 0; r e is then NaN, and
    // the min turns it into q = 1, so the factor 4 r q is 0 as the exact one
    // (4 e^{-2u} there) rounds to.
    __device__ __forceinline__ void r_q(float x, float &r, float &q) const {
        const float e = exp2_fast(x * c2);
        r = rcp_fast(1.0f + e);
        q = fminf(r * e, 1.0f);
    }
    __device__ __forceinline__ static float chain(float r, float q) { return 4.0f * r * q; }
};

// ---- tagged counters -----------------------------------------------------
// Every counter is a 64-bit word: a 32-bit tag above a 32-bit count.  The tag
// of a launch is its dispatch id (the packet's index in its hardware queue,
// which every workgroup of the launch reads from the same SGPRs and every
// launch or graph replay on a queue gets anew) with the top bit set, so no
// launch uses tag 0.  A finished call leaves its words at 0.  At its start,
// each workgroup of a launch claims the words: a compare-and-swap from 0 to
// (tag, 0), issued without waiting for it; the first claim to reach a word
// succeeds and the rest find the tag installed.  Each workgroup's claim is
// ordered before its own draws on the same word (same address, same thread),
// so when the call finds clean words every draw -- a plain increment -- sees
// the launch's tag.  A draw that finds another tag -- a word left by a call
// that never finished, or whatever the workspace held before its first use --
// installs (tag, 1) with a compare-and-swap and takes count 0, or, if another
// workgroup of the launch got there first, draws again.  So the counters never
// need clearing before a call.
}  // namespace dev
extern "C" __device__ unsigned long long lce_dispatch_id() __asm("llvm.amdgcn.dispatch.id");
namespace dev {
__device__ __forceinline__ unsigned launch_tag() {
    return static_cast<unsigned>(lce_dispatch_id()) | 0x80000000u;
}
// install (tag, 0) in a clean word; the result is not waited for
__device__ __forceinline__ void tagged_claim(unsigned long long *w, unsigned tag) {
    unsigned long long clean = 0ull;
    (void)__hip_atomic_compare_exchange_strong(w, &clean, static_cast<unsigned long long>(tag) << 32,
                                               __ATOMIC_RELAXED, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
// The increment, issued now and resolved later (tagged_count).  A wrapping
// increment (never reaching its bound) rather than an add: the compiler rewrites
// a one-lane add into a wave-level form that consumes the result at once, i.e.
// waits right there for every memory operation issued before it, the row
// loads included.
__device__ __forceinline__ unsigned long long tagged_inc(unsigned long long *w) {
    return __builtin_amdgcn_atomic_inc64(reinterpret_cast<unsigned long *>(w), ~0ul, __ATOMIC_RELAXED, "");
}
// the count of a draw whose increment returned `seen`
__device__ __forceinline__ unsigned tagged_count(unsigned long long *w, unsigned long long seen, unsigned tag) {
    if (static_cast<unsigned>(seen >> 32) == tag) return static_cast<unsigned>(seen);
    unsigned long long cur = __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    for (;;) {
        if (static_cast<unsigned>(cur >> 32) == tag) {   // installed by another workgroup: draw again
            cur = tagged_inc(w);
            if (static_cast<unsigned>(cur >> 32) == tag) return static_cast<unsigned>(cur);
            continue;
        }
        if (__hip_atomic_compare_exchange_strong(w, &cur, (static_cast<unsigned long long>(tag) << 32) | 1ull,
                                                 __ATOMIC_RELAXED, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM))
            return 0u;
    }
}
__device__ __forceinline__ unsigned tagged_draw(unsigned long long *w, unsigned tag) {
    return tagged_count(w, tagged_inc(w), tag);
}

// Word 3 of a gfx9-family buffer descriptor: 32-bit data format, no swizzle.
constexpr int kBufferWord3 = 0x00020000;
// Cache-policy bit of buffer loads/stores: non-temporal (streamed once).
constexpr int kNonTemporal = 2;

// A store performed at memory (system scope): another workgroup, on any XCD,
// reads it past its own L2.
__device__ __forceinline__ void store_through(float *p, float v) {
    __hip_atomic_store(reinterpret_cast<unsigned *>(p), __float_as_uint(v), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_SYSTEM);
}

// Row-kernel workspace: the completion counter at byte 0, the row counter at
// byte 64, the counter of the ignored-row chunks at byte 128 (tagged words, one
// per 64-byte line), int64 n_correct partials of the workgroups from byte 256.
constexpr size_t kWsPartials = 256;
__device__ __forceinline__ unsigned long long *ws_ticket(void *ws) { return static_cast<unsigned long long *>(ws); }
__device__ __forceinline__ unsigned long long *ws_rows(void *ws) { return static_cast<unsigned long long *>(ws) + 8; }
__device__ __forceinline__ unsigned long long *ws_zero_chunks(void *ws) {
    return static_cast<unsigned long long *>(ws) + 16;
}
__device__ __forceinline__ long long *ws_correct(void *ws) {
    return reinterpret_cast<long long *>(static_cast<char *>(ws) + kWsPartials);
}

// ---- element access ---------------------------------------------------------

template <bool BF16> struct Elt;

template <> struct Elt<true> {
    static constexpr int E = 8;       // bf16 per 16-byte vector
    static constexpr int bytes = 2;
    static constexpr uint32_t sign_mask = 0x80008000u;   // the sign bits of a packed word
    __device__ __forceinline__ static uint32_t word(const u32x4 &v, int w) {
        return w == 0 ? v.x : w == 1 ? v.y : w == 2 ? v.z : v.w;
    }
    // element e of the vector, widened exactly to fp32 (e is a compile-time constant after unrolling)
    __device__ __forceinline__ static float get(const u32x4 &v, int e) {
        const uint32_t w = word(v, e >> 1);
        return (e & 1) ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16);
    }
    __device__ __forceinline__ static uint32_t pack2(float lo, float hi) {
        typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
        typedef float f2 __attribute__((ext_vector_type(2)));
        f2 f = {lo, hi};
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf2));   // RNE
    }
    __device__ __forceinline__ static u32x4 pack(const float (&g)[8]) {
        return (u32x4){pack2(g[0], g[1]), pack2(g[2], g[3]), pack2(g[4], g[5]), pack2(g[6], g[7])};
    }
    __device__ __forceinline__ static float load_one(const void *base, int64_t idx) {
        const uint16_t b = static_cast<const uint16_t *>(base)[idx];
        return __uint_as_float(static_cast<uint32_t>(b) << 16);
    }
    __device__ __forceinline__ static void store_one(void *base, int64_t idx, float g) {
        static_cast<__bf16 *>(base)[idx] = static_cast<__bf16>(g);   // RNE
    }
    // one element through a buffer descriptor, at element index idx (AUX: cache policy)
    template <int AUX>
    __device__ __forceinline__ static void store_one(__amdgpu_buffer_rsrc_t r, int idx, float g) {
        const __bf16 b = static_cast<__bf16>(g);   // RNE
        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, b), r, idx * 2, 0, AUX);
    }
};

template <> struct Elt<false> {
    static constexpr int E = 4;       // fp32 per 16-byte vector
    static constexpr int bytes = 4;
    static constexpr uint32_t sign_mask = 0x80000000u;
    __device__ __forceinline__ static float get(const u32x4 &v, int e) {
        return __uint_as_float(e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w);
    }
    __device__ __forceinline__ static u32x4 pack(const float (&g)[4]) {
        return (u32x4){__float_as_uint(g[0]), __float_as_uint(g[1]), __float_as_uint(g[2]),
                       __float_as_uint(g[3])};
    }
    __device__ __forceinline__ static float load_one(const void *base, int64_t idx) {
        return static_cast<const float *>(base)[idx];
    }
    __device__ __forceinline__ static void store_one(void *base, int64_t idx, float g) {
        static_cast<float *>(base)[idx] = g;
    }
    template <int AUX>
    __device__ __forceinline__ static void store_one(__amdgpu_buffer_rsrc_t r, int idx, float g) {
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(g), r, idx * 4, 0, AUX);
    }
};

// ---- reductions -------------------------------------------------------------
// Butterfly (xor) shuffles: every lane ends with the same value because each
// step combines the same two operands (IEEE max/add are commutative).

// DPP lane exchanges (VALU, no LDS round trip): within each quad the partner
// at xor 1 and xor 2, then the mirror within each 8 lanes and within each 16
// lanes.  After the four steps every lane of a 16-lane row holds the row's
// combination; the four rows are then read out and combined in a fixed order.
constexpr int kDppXor1 = 0xB1;         // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;  // lane i <-> 7 - i within each 8
constexpr int kDppMirror = 0x140;      // lane i <-> 15 - i within each 16
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) { return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, false); }
__device__ __forceinline__ float lane_f(float v, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

// (m, s) pairs of an online softmax: s is a sum of exponentials relative to m.
__device__ __forceinline__ void lse_combine(float &m, float &s, float m2, float s2) {
    const float mx = fmaxf(m, m2);
    s = s * exp2_fast((m - mx) * kLog2e) + s2 * exp2_fast((m2 - mx) * kLog2e);
    m = mx;
}
template <int CTRL>
__device__ __forceinline__ void lse_step(float &m, float &s) {
    const float m2 = dpp_f<CTRL>(m), s2 = dpp_f<CTRL>(s);
    lse_combine(m, s, m2, s2);
}
// the wave's combined (m, s), the same in every lane
__device__ __forceinline__ void wave_lse(float &m, float &s) {
    lse_step<kDppXor1>(m, s);
    lse_step<kDppXor2>(m, s);
    lse_step<kDppHalfMirror>(m, s);
    lse_step<kDppMirror>(m, s);
    float m0 = lane_f(m, 0), s0 = lane_f(s, 0);
    float m1 = lane_f(m, 32), s1 = lane_f(s, 32);
    lse_combine(m0, s0, lane_f(m, 16), lane_f(s, 16));
    lse_combine(m1, s1, lane_f(m, 48), lane_f(s, 48));
    lse_combine(m0, s0, m1, s1);
    m = m0;
    s = s0;
}
// the wave's sum, the same in every lane
__device__ __forceinline__ float wave_sum_dpp(float v) {
    v += dpp_f<kDppXor1>(v);
    v += dpp_f<kDppXor2>(v);
    v += dpp_f<kDppHalfMirror>(v);
    v += dpp_f<kDppMirror>(v);
    return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

__device__ __forceinline__ long long wave_sum_ll(long long v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// (value, index) order: larger value first, then smaller index.
__device__ __forceinline__ void argmax_combine(float &v, int &i, float v2, int i2) {
    if (v2 > v || (v2 == v && i2 < i)) {
        v = v2;
        i = i2;
    }
}

__device__ __forceinline__ void wave_argmax(float &v, int &i) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float v2 = __shfl_xor(v, o, 64);
        const int i2 = __shfl_xor(i, o, 64);
        argmax_combine(v, i, v2, i2);
    }
}

// the wave's (value, first index), the same in every lane, on the DPP path
template <int CTRL>
__device__ __forceinline__ void argmax_step(float &v, int &i) {
    const float v2 = dpp_f<CTRL>(v);
    const int i2 = dpp_i<CTRL>(i);
    argmax_combine(v, i, v2, i2);
}
__device__ __forceinline__ void wave_argmax_dpp(float &v, int &i) {
    argmax_step<kDppXor1>(v, i);
    argmax_step<kDppXor2>(v, i);
    argmax_step<kDppHalfMirror>(v, i);
    argmax_step<kDppMirror>(v, i);
    float v0 = lane_f(v, 0), v1 = lane_f(v, 32);
    int i0 = __builtin_amdgcn_readlane(i, 0), i1 = __builtin_amdgcn_readlane(i, 32);
    argmax_combine(v0, i0, lane_f(v, 16), __builtin_amdgcn_readlane(i, 16));
    argmax_combine(v1, i1, lane_f(v, 48), __builtin_amdgcn_readlane(i, 48));
    argmax_combine(v0, i0, v1, i1);
    v = v0;
    i = i0;
}

// Block reductions: one LDS slot per wave, then every thread folds the slots
// in wave order, so all threads hold the same result without a second
// barrier.  A call site must not reuse its LDS array before another barrier
// has separated the reads from the next writes.
__device__ __forceinline__ float block_max(float v, float *sh) {
    v = wave_max(v);
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
    __syncthreads();
    float r = sh[0];
#pragma unroll
    for (int w = 1; w < NWAVE; ++w) r = fmaxf(r, sh[w]);
    return r;
}

__device__ __forceinline__ float block_sum(float v, float *sh) {
    v = wave_sum(v);
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
    __syncthreads();
    float r = sh[0];
#pragma unroll
    for (int w = 1; w < NWAVE; ++w) r += sh[w];
    return r;
}

__device__ __forceinline__ void block_argmax(float &v, int &i, float *shv, int *shi) {
    wave_argmax(v, i);
    if ((threadIdx.x & 63) == 0) {
        shv[threadIdx.x >> 6] = v;
        shi[threadIdx.x >> 6] = i;
    }
    __syncthreads();
    v = shv[0];
    i = shi[0];
#pragma unroll
    for (int w = 1; w < NWAVE; ++w) argmax_combine(v, i, shv[w], shi[w]);
}

// Valid-label and bad-label counts over the count labels, by one workgroup.
// Label counting for the mean's denominator, in two halves around a barrier
// of the caller's.  publish: this thread's share of
// count_labels[0, count_n) -- y0 and y1 are its labels at indexes tid and
// tid + NT (ignore_index past count_n), loaded by the caller ahead of its
// other memory traffic, the rest are loaded here -- summed per wave into
// sh[0][wave] (valid) and sh[1][wave] (bad).  read: the totals, once a barrier
// has passed since every wave published.
__device__ __forceinline__ void count_labels_publish(const CEArgs &a, long long (*sh)[NWAVE], int64_t y0, int64_t y1) {
    long long v = 0, b = 0;
    auto count = [&](int64_t y) {
        if (y != a.ignore_index) {
            if (y >= 0 && y < a.V) ++v;
            else ++b;
        }
    };
    count(y0);
    count(y1);
    for (int64_t i = threadIdx.x + 2 * NT; i < a.count_n; i += NT) count(a.count_labels[i]);
    v = wave_sum_ll(v);
    b = wave_sum_ll(b);
    if ((threadIdx.x & 63) == 0) {
        sh[0][threadIdx.x >> 6] = v;
        sh[1][threadIdx.x >> 6] = b;
    }
}
__device__ __forceinline__ void count_labels_read(long long (*sh)[NWAVE], long long &nv, long long &nb) {
    nv = 0;
    nb = 0;
#pragma unroll
    for (int w = 0; w < NWAVE; ++w) {
        nv += sh[0][w];
        nb += sh[1][w];
    }
}

}  // namespace dev
}  // namespace lce
