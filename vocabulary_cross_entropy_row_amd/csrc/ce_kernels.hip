// Cross-entropy forward + backward kernels for gfx950 (CDNA4, wave64).
//
// What is computed (per row i, label y, eps = label smoothing, T = softcap):
//   z      = T > 0 ? T tanh(x / T) : x
//   loss_i = LSE(z) - (1 - eps) z_y - (eps / V) sum_j z_j
//   dx_ij  = s_i (softmax(z)_j - (1 - eps)[j == y] - eps / V) dz_j/dx_j
// following Liger-Kernel PR "Add Megatron-LM cross-entropy integration"
// (Summary: online softmax, gradient written into the logits buffer, no full
// softmax kept; Test setup: the same operation as torch's cross_entropy),
// Megatron-LM PR "Add opt-in Liger vocab-parallel cross entropy" ("What does
// this PR do?": fp32 per-token losses, any upstream gradient, original argmax
// with smallest-index ties) and Liger-Kernel PR "Add Liger Kernel support for
// Muse Glimmer" (Details/Softcap: T tanh(x / T); Summary: token accuracy).
//
// Design (MI355X-first, not a translation of the pages' Triton kernel):
//  * One 1024-thread workgroup per row.  Each thread loads its share of the
//    row with 16-byte non-temporal loads into registers (up to 26 vectors =
//    104 VGPRs), so the row is read from HBM exactly once and written once:
//    2 N V b bytes, the algorithmic minimum for an in-place gradient.
//  * Three passes over the registers: max (+ argmax), sum of exponentials,
//    gradient.  Wave reductions use cross-lane shuffles, LDS only carries the
//    16 per-wave partials between waves.
//  * The target column is left out of the exponential sum, so 1 - p_y is
//    formed as sum_{j != y} e_j / S without cancellation when p_y -> 1.
//  * Ignored rows are never read: their gradient is stored as zeros.
//  * A row that does not fit (odd V, unaligned rows, very wide rows) takes a
//    generic kernel that streams the row from memory three times.
//  * The mean loss is reduced deterministically by the last workgroup to
//    finish (a completion counter in the caller's workspace); n_correct uses
//    integer atomics, which are order-independent.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "lce_internal.h"

namespace lce {
namespace {

// 16-byte vector as a clang vector type (usable with the non-temporal builtins).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int NT = kRowThreads;
constexpr int NWAVE = NT / 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float exp2_fast(float t) { return __builtin_amdgcn_exp2f(t); }

// Hide the register-resident row from the optimiser between passes.  Without
// this the compiler keeps every widened (fp32) element of pass 1 alive for
// reuse in passes 2 and 3, doubling the row's register footprint and spilling.
template <int K>
__device__ __forceinline__ void opaque_row(u32x4 (&v)[K]) {
#pragma unroll
    for (int k = 0; k < K; ++k) asm volatile("" : "+v"(v[k]));
}
__device__ __forceinline__ float rcp_fast(float t) { return __builtin_amdgcn_rcpf(t); }

// Softcap support.  With u = x / T:  tanh(u) = 1 - 2 r,  r = 1 / (1 + e^{2u}),
// so z = T - 2 T r and dz/dx = 1 - tanh^2(u) = 4 r (1 - r).  r is computed from
// the hardware base-2 exponential and reciprocal.
struct Cap {
    float c2;   // 2 log2(e) / T
    float T;
    __device__ __forceinline__ float r_of(float x) const { return rcp_fast(1.0f + exp2_fast(x * c2)); }
    __device__ __forceinline__ float z_of_r(float r) const { return fmaf(-2.0f * T, r, T); }
    __device__ __forceinline__ static float chain_of_r(float r) { return 4.0f * r * (1.0f - r); }
};

// ---- element access ---------------------------------------------------------

template <bool BF16> struct Elt;

template <> struct Elt<true> {
    static constexpr int E = 8;       // bf16 per 16-byte vector
    static constexpr int bytes = 2;
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
        typedef __bf16 bf1;
        static_cast<bf1 *>(base)[idx] = static_cast<bf1>(g);   // RNE
    }
};

template <> struct Elt<false> {
    static constexpr int E = 4;       // fp32 per 16-byte vector
    static constexpr int bytes = 4;
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
};

// ---- reductions -------------------------------------------------------------
// Butterfly (xor) shuffles: every lane ends with the same value because each
// step combines the same two operands (IEEE max/add are commutative).

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

// Block reductions: one LDS slot per wave, then every thread folds the slots
// in wave order, so all threads hold the same result without a second barrier.
// Each call site passes its own LDS array, so no barrier is needed before reuse.
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

// ---- per-row bookkeeping ----------------------------------------------------

struct RowInfo {
    bool valid;
    int y;          // label (0 when invalid)
    float scale;    // d loss_total / d loss_i
};

__device__ __forceinline__ RowInfo row_info(const CEArgs &a, int64_t row) {
    RowInfo r;
    const int64_t y = a.labels[row];
    r.valid = y != a.ignore_index && y >= 0 && y < a.V;
    r.y = r.valid ? static_cast<int>(y) : 0;
    if (a.reduction == 0) {             // none: per-token upstream gradient
        r.scale = a.grad_out ? a.grad_out[row] : 1.0f;
    } else {
        const float g = a.grad_out ? a.grad_out[0] : 1.0f;
        if (a.reduction == 1) {         // mean over valid tokens
            const int64_t nv = a.counts[0];
            r.scale = nv > 0 ? g / static_cast<float>(nv) : 0.0f;
        } else {
            r.scale = g;
        }
    }
    return r;
}

// The last workgroup to finish folds loss_tok into loss_out (fixed order, fp64).
// Only thread 0 wrote anything another workgroup reads (loss_tok[row]), so only
// thread 0 releases; the other waves may retire with their gradient stores
// still in flight.
__device__ void finish_call(const CEArgs &a, int *sh_flag, double *sh_d) {
    if (threadIdx.x == 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        const unsigned t = __hip_atomic_fetch_add(a.ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int last = t == gridDim.x - 1;
        if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        *sh_flag = last;
    }
    __syncthreads();
    if (!*sh_flag) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    double acc = 0.0;
    for (int64_t i = threadIdx.x; i < a.n; i += blockDim.x) acc += static_cast<double>(a.loss_tok[i]);
    acc = wave_sum_d(acc);
    if ((threadIdx.x & 63) == 0) sh_d[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        double tot = 0.0;
        for (int w = 0; w < static_cast<int>(blockDim.x >> 6); ++w) tot += sh_d[w];
        if (a.loss_out) {
            float out = 0.0f;
            if (a.reduction == 1) {
                const int64_t nv = a.counts[0];
                out = nv > 0 ? static_cast<float>(tot / static_cast<double>(nv)) : 0.0f;
            } else if (a.reduction == 2) {
                out = static_cast<float>(tot);
            }
            *a.loss_out = out;
        }
        *a.ticket = 0u;
    }
}

__device__ __forceinline__ void record_argmax(const CEArgs &a, int64_t row, const RowInfo &ri, int am) {
    a.argmax_out[row] = am;
    if (ri.valid && am == ri.y)
        atomicAdd(reinterpret_cast<unsigned long long *>(&a.counts[1]), 1ull);
}

// ---- count kernel -----------------------------------------------------------

__global__ __launch_bounds__(1024) void ce_count_kernel(const int64_t *labels, int64_t n, int64_t V,
                                                        int64_t ignore_index, int64_t *counts,
                                                        unsigned *ticket, float *loss_out) {
    __shared__ long long sh[2][16];
    long long nv = 0, nb = 0;
    for (int64_t i = threadIdx.x; i < n; i += 1024) {
        const int64_t y = labels[i];
        if (y != ignore_index) {
            if (y >= 0 && y < V) ++nv;
            else ++nb;
        }
    }
    nv = wave_sum_ll(nv);
    nb = wave_sum_ll(nb);
    if ((threadIdx.x & 63) == 0) {
        sh[0][threadIdx.x >> 6] = nv;
        sh[1][threadIdx.x >> 6] = nb;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        long long a = 0, b = 0;
        for (int w = 0; w < 16; ++w) {
            a += sh[0][w];
            b += sh[1][w];
        }
        counts[0] = a;
        counts[1] = 0;
        counts[2] = b;
        if (ticket) *ticket = 0u;
        if (loss_out) *loss_out = 0.0f;
    }
}

// ---- register-resident row kernel --------------------------------------------

template <bool BF16, int K, bool SOFTCAP, bool ARGMAX, bool SMOOTH>
__global__ __launch_bounds__(NT) void ce_row_fast(CEArgs a) {
    using EL = Elt<BF16>;
    constexpr int E = EL::E;
    __shared__ float sh_m[NWAVE], sh_s[NWAVE], sh_z[NWAVE];
    __shared__ int sh_i[NWAVE];
    __shared__ int sh_flag;
    __shared__ double sh_d[NWAVE];

    const int tid = threadIdx.x;
    const int64_t row = blockIdx.x;
    const int nvec = static_cast<int>(a.V / E);
    const RowInfo ri = row_info(a, row);
    u32x4 *rp = reinterpret_cast<u32x4 *>(static_cast<char *>(a.logits) + row * a.ld * EL::bytes);
    const u32x4 zero4 = (u32x4){0u, 0u, 0u, 0u};

    if (!ARGMAX && !ri.valid) {
        // an ignored token has a zero gradient and needs no read
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int idx = k * NT + tid;
            if (idx < nvec) __builtin_nontemporal_store(zero4, rp + idx);
        }
        if (tid == 0) a.loss_tok[row] = 0.0f;
        finish_call(a, &sh_flag, sh_d);
        return;
    }

    u32x4 v[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int idx = k * NT + tid;
        v[k] = idx < nvec ? __builtin_nontemporal_load(rp + idx) : zero4;
    }

    // pass 1: row maximum of the raw logits (and its first index)
    float m = -INFINITY;
    int am = 0x7fffffff;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int idx = k * NT + tid;
        if (idx < nvec) {
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const float x = EL::get(v[k], e);
                if constexpr (ARGMAX) {
                    if (x > m) {
                        m = x;
                        am = idx * E + e;
                    }
                } else {
                    m = fmaxf(m, x);
                }
            }
        }
    }
    if constexpr (ARGMAX) {
        block_argmax(m, am, sh_m, sh_i);
        if (tid == 0) record_argmax(a, row, ri, am);
        if (!ri.valid) {
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const int idx = k * NT + tid;
                if (idx < nvec) __builtin_nontemporal_store(zero4, rp + idx);
            }
            if (tid == 0) a.loss_tok[row] = 0.0f;
            finish_call(a, &sh_flag, sh_d);
            return;
        }
    } else {
        m = block_max(m, sh_m);
    }

    const Cap cap{SOFTCAP ? 2.0f * kLog2e / a.softcap : 0.0f, a.softcap};
    const float xy = EL::load_one(a.logits, row * a.ld + ri.y);
    float Mz, zy;
    if constexpr (SOFTCAP) {
        Mz = cap.z_of_r(cap.r_of(m));   // tanh is increasing: max z = cap(max x)
        zy = cap.z_of_r(cap.r_of(xy));
    } else {
        Mz = m;
        zy = xy;
    }
    // where the target element lives: round ky, thread ty, element ey
    const int vy = ri.y / E, ey = ri.y % E, ky = vy / NT, ty = vy % NT;
    const bool owner = tid == ty;

    // pass 2: s = sum_{j != y} exp(z_j - Mz), zs = sum_j z_j
    const float MzL = Mz * kLog2e;
    const float capk = -2.0f * a.softcap * kLog2e;          // d(z log2e)/dr
    const float capb = (a.softcap - Mz) * kLog2e;           // (T - Mz) log2e
    float s = 0.0f, zs = 0.0f;
    opaque_row(v);
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int idx = k * NT + tid;
        if (idx < nvec) {
            float ex[E];
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const float x = EL::get(v[k], e);
                if constexpr (SOFTCAP) {
                    const float r = cap.r_of(x);
                    ex[e] = exp2_fast(fmaf(r, capk, capb));
                    if constexpr (SMOOTH) zs += cap.z_of_r(r);
                } else {
                    ex[e] = exp2_fast(fmaf(x, kLog2e, -MzL));
                    if constexpr (SMOOTH) zs += x;
                }
            }
            if (k == ky) {
#pragma unroll
                for (int e = 0; e < E; ++e)
                    if (owner && e == ey) ex[e] = 0.0f;
            }
            float part = ex[0];
#pragma unroll
            for (int e = 1; e < E; ++e) part += ex[e];
            s += part;
        }
    }
    s = block_sum(s, sh_s);
    if constexpr (SMOOTH) zs = block_sum(zs, sh_z);

    const float eps = a.eps;
    const float invV = 1.0f / static_cast<float>(a.V);
    const float e_y = exp2_fast(fmaf(zy, kLog2e, -MzL));
    const float S = s + e_y;
    const float lse = Mz + logf(S);
    if (tid == 0) {
        float loss = lse - (1.0f - eps) * zy;
        if constexpr (SMOOTH) loss -= eps * invV * zs;
        a.loss_tok[row] = loss;
    }

    // pass 3: gradient, written over the logits
    const float scale = ri.scale;
    const float epsV = SMOOTH ? eps * invV : 0.0f;
    const float lseL = lse * kLog2e;
    const float capb2 = (a.softcap - lse) * kLog2e;
    float gy = scale * (eps - s / S - epsV);                // p_y - (1-eps) - eps/V
    if constexpr (SOFTCAP) gy *= Cap::chain_of_r(cap.r_of(xy));
    opaque_row(v);
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int idx = k * NT + tid;
        if (idx < nvec) {
            float g[E];
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const float x = EL::get(v[k], e);
                if constexpr (SOFTCAP) {
                    const float r = cap.r_of(x);
                    const float p = exp2_fast(fmaf(r, capk, capb2));
                    g[e] = scale * (p - epsV) * Cap::chain_of_r(r);
                } else {
                    const float p = exp2_fast(fmaf(x, kLog2e, -lseL));
                    g[e] = scale * (p - epsV);
                }
            }
            if (k == ky) {
#pragma unroll
                for (int e = 0; e < E; ++e)
                    if (owner && e == ey) g[e] = gy;
            }
            __builtin_nontemporal_store(EL::pack(g), rp + idx);
        }
    }
    finish_call(a, &sh_flag, sh_d);
}

// ---- generic row kernel (any V, any alignment) ------------------------------
// Streams the row from memory three times with element loads.  Used only for
// shapes the register-resident kernel does not take.

template <bool BF16, bool SOFTCAP, bool ARGMAX>
__global__ __launch_bounds__(NT) void ce_row_generic(CEArgs a) {
    using EL = Elt<BF16>;
    __shared__ float sh_m[NWAVE], sh_s[NWAVE], sh_z[NWAVE];
    __shared__ int sh_i[NWAVE];
    __shared__ int sh_flag;
    __shared__ double sh_d[NWAVE];

    const int tid = threadIdx.x;
    const int64_t row = blockIdx.x;
    const int V = static_cast<int>(a.V);
    const RowInfo ri = row_info(a, row);
    const int64_t base = row * a.ld;
    const bool smooth = a.eps != 0.0f;

    float m = -INFINITY;
    int am = 0x7fffffff;
    if (ARGMAX || ri.valid) {
        for (int j = tid; j < V; j += NT) {
            const float x = EL::load_one(a.logits, base + j);
            if constexpr (ARGMAX) {
                if (x > m) {
                    m = x;
                    am = j;
                }
            } else {
                m = fmaxf(m, x);
            }
        }
        if constexpr (ARGMAX) {
            block_argmax(m, am, sh_m, sh_i);
            if (tid == 0) record_argmax(a, row, ri, am);
        } else {
            m = block_max(m, sh_m);
        }
    }
    if (!ri.valid) {
        for (int j = tid; j < V; j += NT) EL::store_one(a.logits, base + j, 0.0f);
        if (tid == 0) a.loss_tok[row] = 0.0f;
        finish_call(a, &sh_flag, sh_d);
        return;
    }

    const Cap cap{SOFTCAP ? 2.0f * kLog2e / a.softcap : 0.0f, a.softcap};
    const float xy = EL::load_one(a.logits, base + ri.y);
    const float Mz = SOFTCAP ? cap.z_of_r(cap.r_of(m)) : m;
    const float zy = SOFTCAP ? cap.z_of_r(cap.r_of(xy)) : xy;
    const float MzL = Mz * kLog2e;
    float s = 0.0f, zs = 0.0f;
    for (int j = tid; j < V; j += NT) {
        const float x = EL::load_one(a.logits, base + j);
        const float z = SOFTCAP ? cap.z_of_r(cap.r_of(x)) : x;
        if (j != ri.y) s += exp2_fast(fmaf(z, kLog2e, -MzL));
        zs += z;
    }
    s = block_sum(s, sh_s);
    zs = block_sum(zs, sh_z);
    const float eps = a.eps;
    const float invV = 1.0f / static_cast<float>(a.V);
    const float S = s + exp2_fast(fmaf(zy, kLog2e, -MzL));
    const float lse = Mz + logf(S);
    if (tid == 0) {
        float loss = lse - (1.0f - eps) * zy;
        if (smooth) loss -= eps * invV * zs;
        a.loss_tok[row] = loss;
    }
    __syncthreads();   // every thread has read x_y before any gradient overwrites it
    const float scale = ri.scale;
    const float epsV = eps * invV;
    const float lseL = lse * kLog2e;
    for (int j = tid; j < V; j += NT) {
        const float x = EL::load_one(a.logits, base + j);
        float g;
        float chain = 1.0f;
        float z = x;
        if constexpr (SOFTCAP) {
            const float r = cap.r_of(x);
            z = cap.z_of_r(r);
            chain = Cap::chain_of_r(r);
        }
        if (j == ri.y) g = scale * (eps - s / S - epsV) * chain;
        else g = scale * (exp2_fast(fmaf(z, kLog2e, -lseL)) - epsV) * chain;
        EL::store_one(a.logits, base + j, g);
    }
    finish_call(a, &sh_flag, sh_d);
}

// ---- read-only argmax kernel --------------------------------------------------

template <bool BF16>
__global__ __launch_bounds__(NT) void ce_argmax_kernel(const void *logits, int64_t ld, int64_t V, bool vec,
                                                       const int64_t *labels, int64_t ignore_index,
                                                       int64_t *argmax_out, int64_t *counts) {
    using EL = Elt<BF16>;
    constexpr int E = EL::E;
    __shared__ float sh_m[NWAVE];
    __shared__ int sh_i[NWAVE];
    const int tid = threadIdx.x;
    const int64_t row = blockIdx.x;
    float m = -INFINITY;
    int am = 0x7fffffff;
    if (vec) {
        const u32x4 *rp = reinterpret_cast<const u32x4 *>(static_cast<const char *>(logits) + row * ld * EL::bytes);
        const int nvec = static_cast<int>(V / E);
        for (int idx = tid; idx < nvec; idx += NT) {
            const u32x4 v = __builtin_nontemporal_load(rp + idx);
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const float x = EL::get(v, e);
                if (x > m) {
                    m = x;
                    am = idx * E + e;
                }
            }
        }
    } else {
        for (int j = tid; j < static_cast<int>(V); j += NT) {
            const float x = EL::load_one(logits, row * ld + j);
            if (x > m) {
                m = x;
                am = j;
            }
        }
    }
    block_argmax(m, am, sh_m, sh_i);
    if (tid == 0) {
        argmax_out[row] = am;
        if (labels) {
            const int64_t y = labels[row];
            if (y != ignore_index && y >= 0 && y < V && am == y)
                atomicAdd(reinterpret_cast<unsigned long long *>(&counts[1]), 1ull);
        }
    }
}

// ---- dispatch ------------------------------------------------------------------

template <bool BF16, int K>
hipError_t launch_fast_k(const CEArgs &a, hipStream_t st) {
    const bool sc = a.softcap > 0.0f, am = a.argmax_out != nullptr, sm = a.eps != 0.0f;
    const dim3 grid(static_cast<unsigned>(a.n)), block(NT);
#define LCE_FAST(S, A, M) hipLaunchKernelGGL((ce_row_fast<BF16, K, S, A, M>), grid, block, 0, st, a)
    if (sc) {
        if (am) { if (sm) LCE_FAST(true, true, true); else LCE_FAST(true, true, false); }
        else    { if (sm) LCE_FAST(true, false, true); else LCE_FAST(true, false, false); }
    } else {
        if (am) { if (sm) LCE_FAST(false, true, true); else LCE_FAST(false, true, false); }
        else    { if (sm) LCE_FAST(false, false, true); else LCE_FAST(false, false, false); }
    }
#undef LCE_FAST
    return hipGetLastError();
}

// Vectors-per-thread instantiations of the register-resident kernel.
constexpr int kKs[] = {1, 2, 4, 8, 12, 16, 20, 24, 26};

template <bool BF16>
hipError_t launch_fast(const CEArgs &a, int k, hipStream_t st) {
    switch (k) {
        case 1: return launch_fast_k<BF16, 1>(a, st);
        case 2: return launch_fast_k<BF16, 2>(a, st);
        case 4: return launch_fast_k<BF16, 4>(a, st);
        case 8: return launch_fast_k<BF16, 8>(a, st);
        case 12: return launch_fast_k<BF16, 12>(a, st);
        case 16: return launch_fast_k<BF16, 16>(a, st);
        case 20: return launch_fast_k<BF16, 20>(a, st);
        case 24: return launch_fast_k<BF16, 24>(a, st);
        case 26: return launch_fast_k<BF16, 26>(a, st);
        default: return hipErrorInvalidValue;
    }
}

template <bool BF16>
hipError_t launch_generic(const CEArgs &a, hipStream_t st) {
    const bool sc = a.softcap > 0.0f, am = a.argmax_out != nullptr;
    const dim3 grid(static_cast<unsigned>(a.n)), block(NT);
    if (sc) {
        if (am) hipLaunchKernelGGL((ce_row_generic<BF16, true, true>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((ce_row_generic<BF16, true, false>), grid, block, 0, st, a);
    } else {
        if (am) hipLaunchKernelGGL((ce_row_generic<BF16, false, true>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((ce_row_generic<BF16, false, false>), grid, block, 0, st, a);
    }
    return hipGetLastError();
}

}  // namespace

int ce_fast_path_k(const void *logits, int64_t ld, bool is_bf16, int64_t V) {
    const int E = is_bf16 ? 8 : 4;
    const int bytes = is_bf16 ? 2 : 4;
    if (V % E != 0 || ld % E != 0) return 0;
    if ((reinterpret_cast<uintptr_t>(logits) & 15u) != 0) return 0;
    (void)bytes;
    const int64_t nvec = V / E;
    const int64_t need = (nvec + NT - 1) / NT;
    for (int k : kKs)
        if (k >= need) return k;
    return 0;
}

hipError_t launch_ce_fwd_bwd(const CEArgs &a, bool is_bf16, hipStream_t stream) {
    hipLaunchKernelGGL(ce_count_kernel, dim3(1), dim3(1024), 0, stream, a.labels, a.n, a.V, a.ignore_index,
                       a.counts, a.ticket, a.loss_out);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || a.n == 0) return err;
    const int k = ce_fast_path_k(a.logits, a.ld, is_bf16, a.V);
    if (k > 0) return is_bf16 ? launch_fast<true>(a, k, stream) : launch_fast<false>(a, k, stream);
    return is_bf16 ? launch_generic<true>(a, stream) : launch_generic<false>(a, stream);
}

hipError_t launch_ce_argmax(const void *logits, int64_t ld, bool is_bf16, const int64_t *labels, int64_t n,
                            int64_t V, int64_t ignore_index, int64_t *argmax_out, int64_t *counts,
                            hipStream_t stream) {
    if (labels) {
        hipLaunchKernelGGL(ce_count_kernel, dim3(1), dim3(1024), 0, stream, labels, n, V, ignore_index, counts,
                           static_cast<unsigned *>(nullptr), static_cast<float *>(nullptr));
    } else {
        hipLaunchKernelGGL(ce_count_kernel, dim3(1), dim3(1024), 0, stream, labels, int64_t(0), V, ignore_index,
                           counts, static_cast<unsigned *>(nullptr), static_cast<float *>(nullptr));
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || n == 0) return err;
    const int E = is_bf16 ? 8 : 4;
    const bool vec = (V % E == 0) && (ld % E == 0) && ((reinterpret_cast<uintptr_t>(logits) & 15u) == 0);
    const dim3 grid(static_cast<unsigned>(n)), block(NT);
    if (is_bf16)
        hipLaunchKernelGGL(ce_argmax_kernel<true>, grid, block, 0, stream, logits, ld, V, vec, labels, ignore_index,
                           argmax_out, counts);
    else
        hipLaunchKernelGGL(ce_argmax_kernel<false>, grid, block, 0, stream, logits, ld, V, vec, labels, ignore_index,
                           argmax_out, counts);
    return hipGetLastError();
}

}  // namespace lce
