// Cross-entropy kernels outside the persistent resident path (gfx950):
//  * ce_count_kernel  - valid / bad label counts (and resets of the call's
//                       outputs) for the generic path and the argmax entry point;
//  * ce_row_generic   - any V, any alignment: streams the row from memory three
//                       times with element loads; used only for shapes the
//                       resident kernel (ce_rows.h) does not take;
//  * ce_argmax_kernel - read-only argmax sweep.
// and the host dispatch between them.  The operation is the one stated in
// ce_rows.h (Liger-Kernel PR "Add Megatron-LM cross-entropy integration",
// Summary; Megatron-LM PR "Add opt-in Liger vocab-parallel cross entropy",
// "What does this PR do?"; Liger-Kernel PR "Add Liger Kernel support for Muse
// Glimmer", Details/Softcap).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "ce_device.h"
#include "lce_internal.h"

namespace lce {
namespace {

using namespace dev;

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
        // the tagged completion counter (see tagged_draw)
        const unsigned t = tagged_draw(ws_ticket(a.workspace), launch_tag());
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
        *ws_ticket(a.workspace) = 0ull;
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
                                                        unsigned long long *ticket, float *loss_out) {
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
        if (ticket) {
            // the row kernel's completion, row and zeroing-chunk counters (tagged,
            // so not required; a clobbered workspace then starts from clean words)
            *ws_ticket(ticket) = 0ull;
            *ws_rows(ticket) = 0ull;
            *ws_zero_chunks(ticket) = 0ull;
        }
        if (loss_out) *loss_out = 0.0f;
    }
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
    if (tid == 0) tagged_claim(ws_ticket(a.workspace), launch_tag());
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
    // every weight relative to the row max itself (z - M is exact where the
    // weight matters), not to an fp32 rounding of M log2 e
    float s = 0.0f, zs = 0.0f;
    for (int j = tid; j < V; j += NT) {
        const float x = EL::load_one(a.logits, base + j);
        const float z = SOFTCAP ? cap.z_of_r(cap.r_of(x)) : x;
        if (j != ri.y) s += exp2_fast((z - Mz) * kLog2e);
        zs += z;
    }
    s = block_sum(s, sh_s);
    zs = block_sum(zs, sh_z);
    const float eps = a.eps;
    const float invV = 1.0f / static_cast<float>(a.V);
    const float S = s + exp2_fast((zy - Mz) * kLog2e);
    const float lse = Mz + logf(S);
    if (tid == 0) {
        float loss = lse - (1.0f - eps) * zy;
        if (smooth) loss -= eps * invV * zs;
        a.loss_tok[row] = loss;
    }
    __syncthreads();   // every thread has read x_y before any gradient overwrites it
    const float scale = ri.scale;
    const float epsV = eps * invV;
    // exponent (z - M) log2 e - log2 S, consistent with the weights above
    const float l2S = log2f(S);
    for (int j = tid; j < V; j += NT) {
        const float x = EL::load_one(a.logits, base + j);
        float g;
        float chain = 1.0f;
        float z = x;
        if constexpr (SOFTCAP) {
            float r, q;
            cap.r_q(x, r, q);
            z = cap.z_of_r(r);
            chain = Cap::chain(r, q);
        }
        if (j == ri.y) g = scale * (eps - s / S - epsV) * chain;
        else g = scale * (exp2_fast(fmaf(z - Mz, kLog2e, -l2S)) - epsV) * chain;
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

// Resident-path families compiled from ce_rows_inst.hip: (register rounds, LDS rounds).
#define LCE_FAMILIES(X) X(1, 0) X(2, 0) X(4, 0) X(8, 0) X(4, 8) X(8, 8) X(10, 9) X(13, 9) X(16, 9)
// The families also built for rows that need not start on a 16-byte boundary
// (rows of up to 16 rounds; wider unaligned rows take the generic kernel).
#define LCE_UA_FAMILIES(X) X(1, 0) X(2, 0) X(4, 0) X(8, 0) X(4, 8) X(8, 8)
#define LCE_DECL(kr, kl)                                                           \
    hipError_t launch_rows_0_0_##kr##_##kl(const CEArgs &, int, hipStream_t);     \
    hipError_t launch_rows_0_1_##kr##_##kl(const CEArgs &, int, hipStream_t);
LCE_FAMILIES(LCE_DECL)
#undef LCE_DECL
#define LCE_UA_DECL(kr, kl)                                                        \
    hipError_t launch_rows_1_0_##kr##_##kl(const CEArgs &, int, hipStream_t);     \
    hipError_t launch_rows_1_1_##kr##_##kl(const CEArgs &, int, hipStream_t);
LCE_UA_FAMILIES(LCE_UA_DECL)
#undef LCE_UA_DECL

// Short-row families compiled from ce_rows_mr.hip: (waves per row, vectors per lane).
#define LCE_MR_FAMILIES(X) X(1, 1) X(1, 2) X(1, 4) X(1, 8) X(2, 8) X(4, 8) X(4, 16)
#define LCE_MR_DECL(p, kv)                                                          \
    hipError_t launch_rows_mr_0_##p##_##kv(const CEArgs &, int, hipStream_t);      \
    hipError_t launch_rows_mr_1_##p##_##kv(const CEArgs &, int, hipStream_t);
LCE_MR_FAMILIES(LCE_MR_DECL)
#undef LCE_MR_DECL

// Half-row families compiled from ce_rows_half.hip: rounds of 960 vectors per half row.
#define LCE_HALF_FAMILIES(X) X(5) X(6) X(7) X(8) X(9) X(10)
#define LCE_HALF_DECL(kh)                                                       \
    hipError_t launch_rows_half_0_##kh(const CEArgs &, int, hipStream_t);      \
    hipError_t launch_rows_half_1_##kh(const CEArgs &, int, hipStream_t);
LCE_HALF_FAMILIES(LCE_HALF_DECL)
#undef LCE_HALF_DECL

// Rows of at most this many 16-byte vectors go to the short-row kernel.
constexpr int64_t kMrMaxVectors = 4096;

bool ce_short_plan(const void *logits, int64_t ld, bool is_bf16, int64_t n, int64_t V, int *p, int *kv) {
    const int E = is_bf16 ? 8 : 4;
    if (V % E != 0 || ld % E != 0) return false;
    if ((reinterpret_cast<uintptr_t>(logits) & 15u) != 0) return false;
    const int64_t nvec = V / E;
    if (nvec > kMrMaxVectors) return false;
    // rows of 2049-4096 vectors (four waves of 16 vectors a lane) only while a CU sees few rows:
    // 2048 x 32768 55.6 against 59.0 us per call with the persistent row kernel, 8192 x 32768 199
    // against 180 us
    if (nvec > 2048 && n > 4096) return false;
#define LCE_MR_ENTRY(a, b) {a, b},
    static const int fam[][2] = {LCE_MR_FAMILIES(LCE_MR_ENTRY)};   // in increasing capacity
#undef LCE_MR_ENTRY
    for (const auto &f : fam)
        if (64 * f[0] * f[1] >= nvec) {
            *p = f[0];
            *kv = f[1];
            return true;
        }
    return false;
}

bool ce_resident_plan(const void *logits, int64_t ld, bool is_bf16, int64_t V, int *kr, int *kl, bool *ua) {
    const int E = is_bf16 ? 8 : 4;
    // rows on 16-byte boundaries, or else read through aligned windows of up to
    // one more vector
    *ua = V % E != 0 || ld % E != 0 || (reinterpret_cast<uintptr_t>(logits) & 15u) != 0;
    const int64_t nv = *ua ? (V + 2 * E - 2) / E : V / E;
    const int64_t need = (nv + NT - 1) / NT;   // rounds of 1024 vectors
#define LCE_FAM_ENTRY(r, l) {r, l},
    static const int fam[][2] = {LCE_FAMILIES(LCE_FAM_ENTRY)};        // in increasing K = KR + KL
    static const int fam_ua[][2] = {LCE_UA_FAMILIES(LCE_FAM_ENTRY)};
#undef LCE_FAM_ENTRY
    if (*ua) {
        for (const auto &f : fam_ua)
            if (f[0] + f[1] >= need) {
                *kr = f[0];
                *kl = f[1];
                return true;
            }
        return false;
    }
    for (const auto &f : fam)
        if (f[0] + f[1] >= need) {
            *kr = f[0];
            *kl = f[1];
            return true;
        }
    return false;
}

bool ce_half_plan(const void *logits, int64_t ld, bool is_bf16, int64_t n, int64_t V, int *kh) {
    const int E = is_bf16 ? 8 : 4;
    if (V % E != 0 || ld % E != 0 || n < 1 || n > 0x7fffffffLL) return false;
    if ((reinterpret_cast<uintptr_t>(logits) & 15u) != 0) return false;
    const int64_t hv0 = (V / E + 1) / 2;
    const int64_t need = (hv0 + 959) / 960;   // rounds of 960 vectors per half row
#define LCE_HALF_ENTRY(k) k,
    static const int fam[] = {LCE_HALF_FAMILIES(LCE_HALF_ENTRY)};
#undef LCE_HALF_ENTRY
    // Half rows of 6-8 rounds beat the persistent row kernel at any row count (2048 x 92160: 143 against
    // 152 us per call, 8192 x 100352: 552 against 562-579 us; 8 rounds about even), those of 5 rounds
    // only while a CU sees few rows (2048 x 65536: 100.8 against 104.4 us); with 32 rows per CU the
    // persistent kernel's dynamic walk is as fast there.
    if (need == 5 && n > 4096) return false;
    for (int f : fam)
        if (f == need) {
            *kh = f;
            return true;
        }
    return false;
}

int device_cu_count() {
    static int cus[64] = {0};
    int d = 0;
    if (hipGetDevice(&d) != hipSuccess || d < 0 || d >= 64) return 256;
    if (cus[d] == 0) {
        int c = 0;
        if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, d) != hipSuccess || c < 1) c = 256;
        cus[d] = c;
    }
    return cus[d];
}

namespace {

hipError_t launch_resident(const CEArgs &a, bool bf16, int kr, int kl, bool ua, hipStream_t st) {
    const int cus = device_cu_count();
    if (ua) {
#define LCE_UA_CASE(r, l)                                                                                    \
    if (kr == r && kl == l) return bf16 ? launch_rows_1_1_##r##_##l(a, cus, st) : launch_rows_1_0_##r##_##l(a, cus, st);
        LCE_UA_FAMILIES(LCE_UA_CASE)
#undef LCE_UA_CASE
        return hipErrorInvalidValue;
    }
#define LCE_CASE(r, l)                                                                                       \
    if (kr == r && kl == l) return bf16 ? launch_rows_0_1_##r##_##l(a, cus, st) : launch_rows_0_0_##r##_##l(a, cus, st);
    LCE_FAMILIES(LCE_CASE)
#undef LCE_CASE
    return hipErrorInvalidValue;
}
}  // namespace

// The half-row kernel's grid: one 1024-thread workgroup per CU (its LDS slot
// takes most of a CU's LDS), an even count, at most two per row.
hipError_t launch_half(const CEArgs &a, bool bf16, int kh, hipStream_t st) {
    int64_t g = device_cu_count() & ~1;
    if (g > kHalfMaxGroups) g = kHalfMaxGroups;
    if (g > 2 * a.n) g = 2 * a.n;
    if (g < 2) g = 2;
    const int groups = static_cast<int>(g);
#define LCE_HALF_CASE(k) \
    if (kh == k) return bf16 ? launch_rows_half_1_##k(a, groups, st) : launch_rows_half_0_##k(a, groups, st);
    LCE_HALF_FAMILIES(LCE_HALF_CASE)
#undef LCE_HALF_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_short(const CEArgs &a, bool bf16, int p, int kv, hipStream_t st) {
    const int cus = device_cu_count();
#define LCE_MR_CASE(pp, kk)                                                                                  \
    if (p == pp && kv == kk)                                                                                 \
        return bf16 ? launch_rows_mr_1_##pp##_##kk(a, cus, st) : launch_rows_mr_0_##pp##_##kk(a, cus, st);
    LCE_MR_FAMILIES(LCE_MR_CASE)
#undef LCE_MR_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_ce_fwd_bwd(const CEArgs &a, bool is_bf16, hipStream_t stream) {
    int kr = 0, kl = 0, p = 0, kv = 0;
    if (a.n > 0 && ce_short_plan(a.logits, a.ld, is_bf16, a.n, a.V, &p, &kv)) {
        // one launch: the short-row kernel counts labels and reduces on its own
        return launch_short(a, is_bf16, p, kv, stream);
    }
    int kh = 0;
    if (a.n > 0 && ce_half_plan(a.logits, a.ld, is_bf16, a.n, a.V, &kh)) {
        // one launch: pairs of workgroups, one half row each
        return launch_half(a, is_bf16, kh, stream);
    }
    bool ua = false;
    if (a.n > 0 && ce_resident_plan(a.logits, a.ld, is_bf16, a.V, &kr, &kl, &ua)) {
        // one launch: the persistent kernel counts labels and reduces on its own
        return launch_resident(a, is_bf16, kr, kl, ua, stream);
    }
    hipLaunchKernelGGL(ce_count_kernel, dim3(1), dim3(1024), 0, stream, a.count_labels, a.count_n, a.V,
                       a.ignore_index, a.counts, static_cast<unsigned long long *>(a.workspace), a.loss_out);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || a.n == 0) return err;
    return is_bf16 ? launch_generic<true>(a, stream) : launch_generic<false>(a, stream);
}

hipError_t launch_ce_count(const int64_t *labels, int64_t n, int64_t V, int64_t ignore_index, int64_t *counts,
                           unsigned long long *ticket, float *loss_out, hipStream_t stream) {
    hipLaunchKernelGGL(ce_count_kernel, dim3(1), dim3(1024), 0, stream, labels, n, V, ignore_index, counts, ticket,
                       loss_out);
    return hipGetLastError();
}

hipError_t launch_ce_argmax(const void *logits, int64_t ld, bool is_bf16, const int64_t *labels, int64_t n,
                            int64_t V, int64_t ignore_index, int64_t *argmax_out, int64_t *counts,
                            hipStream_t stream) {
    if (labels) {
        hipLaunchKernelGGL(ce_count_kernel, dim3(1), dim3(1024), 0, stream, labels, n, V, ignore_index, counts,
                           static_cast<unsigned long long *>(nullptr), static_cast<float *>(nullptr));
    } else {
        hipLaunchKernelGGL(ce_count_kernel, dim3(1), dim3(1024), 0, stream, labels, int64_t(0), V, ignore_index,
                           counts, static_cast<unsigned long long *>(nullptr), static_cast<float *>(nullptr));
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
