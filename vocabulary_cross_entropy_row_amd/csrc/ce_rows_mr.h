// Cross-entropy row kernel for short rows (gfx950): several rows per workgroup.
//
// The operation is that of ce_rows.h (Liger-Kernel PR "Add Megatron-LM
// cross-entropy integration", Summary and Test setup; Megatron-LM PR "Add
// opt-in Liger vocab-parallel cross entropy", "What does this PR do?";
// Liger-Kernel PR "Add Liger Kernel support for Muse Glimmer",
// Details/Softcap), with the same per-element arithmetic.
//
// Layout of the work: a row of at most 4096 16-byte vectors (bf16 V <= 32768,
// fp32 V <= 16384) is held by P waves, KV vectors per lane, in VGPRs; a
// 512-thread workgroup (8 waves, two per CU) holds 8 / P rows at a time.
// With all 1024 threads on one row, as the long-row kernel does, a row this
// short keeps most threads idle and pays a workgroup-wide combine per few
// kilobytes.  Here a row's statistics combine with DPP exchanges inside its
// waves, plus (P > 1) one LDS exchange between its waves per row step; with
// P = 1 the waves never wait for each other inside the row loop.  Row sets are
// walked statically (workgroup b takes row sets b, b + G, ...).  Two workgroups
// per CU: while one waits for its row set's loads the other computes and
// stores (one 1024-thread workgroup per CU was 3-6% slower on 134 MB calls);
// few enough that every workgroup counting all the labels stays cheap.
//
// Every workgroup counts the labels itself first (the mean's scale needs
// n_valid before any gradient is written; the labels are read from L2).  The
// last workgroup to finish (a tagged completion counter) sums the per-token
// losses in row order in fp64 and the workgroups' n_correct partials, so the
// reductions do not depend on which workgroup took which rows.
#pragma once

#include "ce_device.h"

namespace lce {
namespace dev {

#ifndef LCE_MR_THREADS
#define LCE_MR_THREADS 512
#endif
constexpr int kMrThreads = LCE_MR_THREADS;
constexpr int kMrWaves = kMrThreads / 64;

template <bool BF16, int P, int KV, bool SOFTCAP, bool ARGMAX, bool SMOOTH>
__global__ __launch_bounds__(kMrThreads) __attribute__((amdgpu_waves_per_eu(4))) void ce_rows_mr_kernel(CEArgs a) {
    using EL = Elt<BF16>;
    constexpr int E = EL::E;
    constexpr int R = kMrWaves / P;      // rows per workgroup step
    constexpr int GT = 64 * P;           // threads per row
    // per-row combine slots (P > 1), double-buffered by step parity
    __shared__ float sh_m[2][R][P], sh_s[2][R][P], sh_zs[2][R][P], sh_av[2][R][P];
    __shared__ int sh_ai[2][R][P];
    __shared__ float sh_xy[2][R];
    __shared__ double sh_d[kMrWaves];
    __shared__ long long sh_c[3][kMrWaves];   // valid / bad label counts, n_correct partials
    __shared__ int sh_flag;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: row numbers stay in SGPRs
    const int grp = wave / P;            // row group of this wave
    const int gl = tid - grp * GT;       // lane within the row group
    const int nvec = static_cast<int>(a.V / E);
    const int64_t n = a.n;
    const int64_t G = gridDim.x;
    const float eps = a.eps;
    const float invV = 1.0f / static_cast<float>(a.V);
    const Cap cap{SOFTCAP ? 2.0f * kLog2e / a.softcap : 0.0f, a.softcap};
    const float capk = -2.0f * a.softcap * kLog2e;
    const u32x4 zero4 = {0u, 0u, 0u, 0u};
    typedef const __attribute__((address_space(4))) int64_t *clabels_t;
    typedef const __attribute__((address_space(4))) float *cfloat_t;
    const clabels_t lab = (clabels_t)a.labels;
    const cfloat_t gout = (cfloat_t)a.grad_out;
    const unsigned tag = launch_tag();
    auto valid_label = [&](int64_t y) { return y != a.ignore_index && y >= 0 && y < a.V; };

    // The label counts: kFold labels per thread in flight, then one LDS exchange.
    // The first batch of labels is requested first, then this workgroup's first
    // row set, so counting that batch waits for its own loads only and the row
    // loads overlap the count.
    constexpr int kFold = 8;
    const uint32_t row_bytes = static_cast<uint32_t>(nvec) * 16u;
    int64_t yl0[kFold];
#pragma unroll
    for (int u = 0; u < kFold; ++u) {
        const int64_t i = u * kMrThreads + tid;
        yl0[u] = i < a.count_n ? a.count_labels[i] : a.ignore_index;
    }
    __builtin_amdgcn_sched_barrier(0);
    u32x4 v[KV];
    {
        const int64_t row = static_cast<int64_t>(blockIdx.x) * R + grp;
        const bool live = row < n;
        const int64_t y64 = live ? lab[row] : a.ignore_index;
        const bool read = live && (ARGMAX || valid_label(y64));
        const __amdgpu_buffer_rsrc_t rr = __builtin_amdgcn_make_buffer_rsrc(
            static_cast<char *>(a.logits) + (read ? row : 0) * a.ld * EL::bytes, 0, read ? row_bytes : 0u,
            kBufferWord3);
#pragma unroll
        for (int k = 0; k < KV; ++k)
            v[k] = __builtin_amdgcn_raw_buffer_load_b128(rr, (gl + k * GT) * 16, 0, kNonTemporal);
    }
    __builtin_amdgcn_sched_barrier(0);
    long long n_valid = 0, n_bad = 0;
    {
        long long cv = 0, cb = 0;
        for (int64_t i0 = 0; i0 < a.count_n; i0 += kFold * kMrThreads) {
            int64_t yl[kFold];
#pragma unroll
            for (int u = 0; u < kFold; ++u) {
                const int64_t i = i0 + u * kMrThreads + tid;
                yl[u] = i0 == 0 ? yl0[u] : (i < a.count_n ? a.count_labels[i] : a.ignore_index);
            }
#pragma unroll
            for (int u = 0; u < kFold; ++u)
                if (yl[u] != a.ignore_index) {
                    if (yl[u] >= 0 && yl[u] < a.V) ++cv;
                    else ++cb;
                }
        }
        cv = wave_sum_ll(cv);
        cb = wave_sum_ll(cb);
        if ((tid & 63) == 0) {
            sh_c[0][wave] = cv;
            sh_c[1][wave] = cb;
        }
        __syncthreads();
#pragma unroll
        for (int w = 0; w < kMrWaves; ++w) {
            n_valid += sh_c[0][w];
            n_bad += sh_c[1][w];
        }
    }
    const float g_all = (a.reduction != 0 && gout) ? gout[0] : 1.0f;
    const float red_scale = a.reduction == 1 ? (n_valid > 0 ? g_all / static_cast<float>(n_valid) : 0.0f) : g_all;
    long long correct = 0;

    int pb = 0;
    for (int64_t base = static_cast<int64_t>(blockIdx.x) * R; base < n; base += G * R, pb ^= 1) {
        const int64_t row = base + grp;
        const bool live = row < n;
        const int64_t y64 = live ? lab[row] : a.ignore_index;
        const bool valid = valid_label(y64);
        const bool read = live && (ARGMAX || valid);
        const int y = valid ? static_cast<int>(y64) : 0;
        const float scale = !valid ? 0.0f : (a.reduction == 0 ? (gout ? gout[row] : 1.0f) : red_scale);
        const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(
            static_cast<char *>(a.logits) + (live ? row : 0) * a.ld * EL::bytes, 0, live ? row_bytes : 0u,
            kBufferWord3);
        const __amdgpu_buffer_rsrc_t rr = __builtin_amdgcn_make_buffer_rsrc(
            static_cast<char *>(a.logits) + (read ? row : 0) * a.ld * EL::bytes, 0, read ? row_bytes : 0u,
            kBufferWord3);
        if (base != static_cast<int64_t>(blockIdx.x) * R) {   // the first set's rows were requested above
#pragma unroll
            for (int k = 0; k < KV; ++k)
                v[k] = __builtin_amdgcn_raw_buffer_load_b128(rr, (gl + k * GT) * 16, 0, kNonTemporal);
        }
        const int vy = y / E, ey = y % E, ky = vy / GT, ty = vy % GT;
        const bool owner = gl == ty;

        // ---- pass A: online softmax, argmax, sum z; the target kept out of s
        float m = -FLT_MAX, s = 0.0f, zs = 0.0f, amv = -INFINITY, xy = 0.0f;
        int am_k = -1, am_e = 0;
#pragma unroll
        for (int k = 0; k < KV; ++k) {
            if ((k + 1) * GT <= nvec || gl + k * GT < nvec) {
                float x[E], z[E];
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    x[e] = EL::get(v[k], e);
                    z[e] = SOFTCAP ? cap.r_of(x[e]) : x[e];
                }
                float rmax = z[0];
#pragma unroll
                for (int e = 1; e < E; ++e) rmax = SOFTCAP ? fminf(rmax, z[e]) : fmaxf(rmax, z[e]);
                if constexpr (SOFTCAP) rmax = cap.z_of_r(rmax);
                if constexpr (ARGMAX) {
                    float xmax = x[0];
                    if constexpr (SOFTCAP) {
#pragma unroll
                        for (int e = 1; e < E; ++e) xmax = fmaxf(xmax, x[e]);
                    } else {
                        xmax = rmax;
                    }
                    if (xmax > amv) {
                        int first = E - 1;
#pragma unroll
                        for (int e = E - 2; e >= 0; --e)
                            if (x[e] == xmax) first = e;
                        amv = xmax;
                        am_k = k;
                        am_e = first;
                    }
                }
                if constexpr (SMOOTH) {
                    float t = z[0];
#pragma unroll
                    for (int e = 1; e < E; ++e) t += z[e];
                    zs += SOFTCAP ? fmaf(-2.0f * a.softcap, t, E * a.softcap) : t;
                }
                const float mn = fmaxf(m, rmax);
                const float mnL = mn * kLog2e;
                float ex[E];
                if constexpr (SOFTCAP) {
                    const float b = fmaf(a.softcap, kLog2e, -mnL);
#pragma unroll
                    for (int e = 0; e < E; ++e) ex[e] = exp2_fast(fmaf(z[e], capk, b));
                } else if constexpr (BF16) {
#pragma unroll
                    for (int e = 0; e < E; ++e) ex[e] = exp2_fast(fmaf(z[e], kLog2e, -mnL));
                } else {
#pragma unroll
                    for (int e = 0; e < E; ++e) ex[e] = exp2_fast((z[e] - mn) * kLog2e);
                }
                if (k == ky && owner) {
#pragma unroll
                    for (int e = 0; e < E; ++e)
                        if (e == ey) {
                            xy = x[e];
                            ex[e] = 0.0f;
                        }
                }
                float part = ex[0];
#pragma unroll
                for (int e = 1; e < E; ++e) part += ex[e];
                s = fmaf(s, exp2_fast(BF16 || SOFTCAP ? fmaf(m, kLog2e, -mnL) : (m - mn) * kLog2e), part);
                m = mn;
            }
        }
        // the row's combine: inside each wave by DPP, then (P > 1) across its waves through LDS
        int am = 0x7fffffff;
        wave_lse(m, s);
        if constexpr (ARGMAX) {
            am = am_k < 0 ? 0x7fffffff : ((am_k * GT + gl) * E + am_e);
            wave_argmax_dpp(amv, am);
        }
        if constexpr (SMOOTH) zs = wave_sum_dpp(zs);
        // the target's raw value: from its owner lane (its wave when P > 1)
        if constexpr (P == 1) {
            xy = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, xy), ty));
        } else {
            if (owner) sh_xy[pb][grp] = xy;
            if ((tid & 63) == 0) {
                const int w = wave - grp * P;
                sh_m[pb][grp][w] = m;
                sh_s[pb][grp][w] = s;
                if constexpr (ARGMAX) {
                    sh_av[pb][grp][w] = amv;
                    sh_ai[pb][grp][w] = am;
                }
                if constexpr (SMOOTH) sh_zs[pb][grp][w] = zs;
            }
            __syncthreads();
            float M = sh_m[pb][grp][0];
#pragma unroll
            for (int w = 1; w < P; ++w) M = fmaxf(M, sh_m[pb][grp][w]);
            float S0 = 0.0f;
#pragma unroll
            for (int w = 0; w < P; ++w) S0 += sh_s[pb][grp][w] * exp2_fast((sh_m[pb][grp][w] - M) * kLog2e);
            m = M;
            s = S0;
            if constexpr (ARGMAX) {
                amv = sh_av[pb][grp][0];
                am = sh_ai[pb][grp][0];
#pragma unroll
                for (int w = 1; w < P; ++w) argmax_combine(amv, am, sh_av[pb][grp][w], sh_ai[pb][grp][w]);
            }
            if constexpr (SMOOTH) {
                float t = sh_zs[pb][grp][0];
#pragma unroll
                for (int w = 1; w < P; ++w) t += sh_zs[pb][grp][w];
                zs = t;
            }
            xy = sh_xy[pb][grp];
        }
        if constexpr (ARGMAX)
            if (gl == 0 && live && valid && am == y) ++correct;
        const float Mz = m;
        const float zy = SOFTCAP ? cap.z_of_r(cap.r_of(xy)) : xy;
        const float S = s + exp2_fast((zy - Mz) * kLog2e);
        const float lse = Mz + logf(S);
        float loss = lse - (1.0f - eps) * zy;
        if constexpr (SMOOTH) loss -= eps * invV * zs;
        if (!valid) loss = 0.0f;
        // the row outputs go out before the gradient stores, and in the last row set
        // also this workgroup's n_correct partial: the completion ticket then waits
        // for these, not for the gradient (see the end of the kernel)
        if (live && gl == 0) {
            store_through(a.loss_tok + row, loss);
            if constexpr (ARGMAX) a.argmax_out[row] = am;
        }
        if (base + G * R >= n) {   // this workgroup's last row set (uniform)
            if constexpr (ARGMAX) correct = wave_sum_ll(correct);
            if ((tid & 63) == 0) sh_c[2][wave] = ARGMAX ? correct : 0;
            __syncthreads();
            if (tid == 0) {
                long long c = 0;
#pragma unroll
                for (int w = 0; w < kMrWaves; ++w) c += sh_c[2][w];
                __hip_atomic_store(ws_correct(a.workspace) + blockIdx.x, c, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_SYSTEM);
            }
        }
        asm volatile("" ::: "memory");   // keep those stores ahead of the gradient's

        // ---- pass B: the gradient (the same evaluation as the long-row kernel)
        const float ascale = fabsf(scale);
        const bool negate = scale < 0.0f;
        const float l2s = log2f(ascale);
        const float epsV = SMOOTH ? eps * invV * ascale : 0.0f;
        const float lseL = lse * kLog2e - l2s;
        const float l2rel = l2s - log2f(S);
        const float capb2 = (a.softcap - lse) * kLog2e + l2s;
        float gy = scale * (eps - s / S - (SMOOTH ? eps * invV : 0.0f));
        if constexpr (SOFTCAP) {
            float ry, qy;
            cap.r_q(xy, ry, qy);
            gy *= Cap::chain(ry, qy);
        }
        if (!valid) gy = 0.0f;
        opaque_regs(v);   // re-widen the row in pass B instead of keeping pass A's fp32 copies live
#pragma unroll
        for (int k = 0; k < KV; ++k) {
            u32x4 out = zero4;
            if (valid) {
                float g[E];
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const float x = EL::get(v[k], e);
                    if constexpr (SOFTCAP) {
                        float r, q;
                        cap.r_q(x, r, q);
                        const float p4 = exp2_fast(fmaf(r, capk, capb2 + 2.0f));
                        g[e] = (SMOOTH ? p4 - 4.0f * epsV : p4) * (r * q);
                    } else {
                        const float p = BF16 ? exp2_fast(fmaf(x, kLog2e, -lseL))
                                             : exp2_fast(fmaf(x - Mz, kLog2e, l2rel));
                        g[e] = SMOOTH ? p - epsV : p;
                    }
                    if (negate) g[e] = -g[e];
                }
                out = EL::pack(g);
            }
            // lanes past the row fall outside the descriptor and store nothing; the round
            // offset rides in the VGPR offset (see the long-row kernel's store_round)
            int vo = (gl + k * GT) * 16;
            asm volatile("" : "+v"(vo));
            __builtin_amdgcn_raw_buffer_store_b128(out, rp, vo, 0, kNonTemporal);
        }
        // the target element's own gradient (same thread, same address, after its vector)
        if (live && valid && owner) EL::template store_one<kNonTemporal>(rp, y, gy);
    }

    // ---- the ticket; the last workgroup folds the per-token losses and the
    // n_correct partials.  Those were stored at system scope ahead of the last row
    // set's KV gradient stores (and the target element's one), and a wave's
    // memory operations complete in issue order, so once at most KV of this wave's
    // are outstanding its share has landed; the gradient stores drain meanwhile.
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(KV) : "memory");
    __syncthreads();
    if (tid == 0) {
        tagged_claim(ws_ticket(a.workspace), tag);
        const unsigned t = tagged_draw(ws_ticket(a.workspace), tag);
        sh_flag = t == static_cast<unsigned>(G) - 1u;
    }
    __syncthreads();
    if (!sh_flag) return;
    // fixed order: thread t sums rows t, t + 256, ... in fp64 (kFold loads in flight), then the
    // waves' sums in wave order
    double acc = 0.0;
    // this thread's first n_correct partial goes out with the first batch of losses
    // (clamped like them, masked when added)
    long long cor = __hip_atomic_load(ws_correct(a.workspace) + (tid < G ? tid : 0), __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_SYSTEM);
    for (int64_t r0 = 0; r0 < n; r0 += kFold * kMrThreads) {
        float lv[kFold];
#pragma unroll
        for (int u = 0; u < kFold; ++u) {
            const int64_t r = r0 + u * kMrThreads + tid;
            lv[u] = __uint_as_float(__hip_atomic_load(reinterpret_cast<unsigned *>(a.loss_tok) + (r < n ? r : n - 1),
                                                      __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM));
        }
#pragma unroll
        for (int u = 0; u < kFold; ++u)
            if (r0 + u * kMrThreads + tid < n) acc += static_cast<double>(lv[u]);
    }
    if (tid >= G) cor = 0;
    for (int64_t w = tid + kMrThreads; w < G; w += kMrThreads)
        cor += __hip_atomic_load(ws_correct(a.workspace) + w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    acc = wave_sum_d(acc);
    cor = wave_sum_ll(cor);
    if ((tid & 63) == 0) {
        sh_d[wave] = acc;
        sh_c[2][wave] = cor;
    }
    __syncthreads();
    if (tid == 0) {
        double tot = 0.0;
        long long c = 0;
        for (int w = 0; w < kMrWaves; ++w) {
            tot += sh_d[w];
            c += sh_c[2][w];
        }
        if (a.loss_out) {
            float out = 0.0f;
            if (a.reduction == 1) out = n_valid > 0 ? static_cast<float>(tot / static_cast<double>(n_valid)) : 0.0f;
            else if (a.reduction == 2) out = static_cast<float>(tot);
            *a.loss_out = out;
        }
        a.counts[0] = n_valid;
        a.counts[1] = c;
        a.counts[2] = n_bad;
        // a finished call leaves every counter word of the workspace clear
        *ws_ticket(a.workspace) = 0ull;
        *ws_rows(a.workspace) = 0ull;
        *ws_zero_chunks(a.workspace) = 0ull;
    }
}

// One (dtype, P, KV) family: picks the feature variant and sizes the grid to the
// workgroups the CUs hold at once (or fewer when there are fewer row sets).
template <bool BF16, int P, int KV, bool S, bool A, bool M>
hipError_t launch_mr_variant(const CEArgs &a, int cus, hipStream_t st) {
    static int per_cu = 0;
    if (per_cu == 0) {
        int nb = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, ce_rows_mr_kernel<BF16, P, KV, S, A, M>, kMrThreads, 0) !=
                hipSuccess || nb < 1)
            nb = 1;
        per_cu = nb;
    }
    constexpr int R = kMrWaves / P;
    int64_t grid = static_cast<int64_t>(cus) * per_cu;
    const int64_t sets = (a.n + R - 1) / R;
    if (grid > sets) grid = sets;
    hipLaunchKernelGGL((ce_rows_mr_kernel<BF16, P, KV, S, A, M>), dim3(static_cast<unsigned>(grid)), dim3(kMrThreads),
                       0, st, a);
    return hipGetLastError();
}

template <bool BF16, int P, int KV>
hipError_t launch_rows_mr(const CEArgs &a, int cus, hipStream_t st) {
    const bool sc = a.softcap > 0.0f, am = a.argmax_out != nullptr, sm = a.eps != 0.0f;
#define LCE_MR(S, A, M) return launch_mr_variant<BF16, P, KV, S, A, M>(a, cus, st)
    if (sc) {
        if (am) { if (sm) LCE_MR(true, true, true); else LCE_MR(true, true, false); }
        else    { if (sm) LCE_MR(true, false, true); else LCE_MR(true, false, false); }
    } else {
        if (am) { if (sm) LCE_MR(false, true, true); else LCE_MR(false, true, false); }
        else    { if (sm) LCE_MR(false, false, true); else LCE_MR(false, false, false); }
    }
#undef LCE_MR
}

}  // namespace dev
}  // namespace lce
