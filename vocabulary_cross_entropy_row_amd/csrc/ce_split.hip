// Cross-entropy split into three phases, for a vocabulary split across
// devices (Megatron-LM PR "Add opt-in Liger vocab-parallel cross entropy",
// What does this PR do?: per-token fp32 losses, the supplied TP group, the
// original global argmax with smallest-index ties) and for a backward pass
// whose upstream gradient is known only later (the pages' in-place kernels
// compute the gradient inside the forward; Liger-Kernel PR "[Megatron] Add
// SwiGLU integration", Known issues, is what that costs a reused graph):
//
//   stats    one read of a shard [n, Vs] of the logits (global columns
//            [v0, v0 + Vs)): per row m = max z, s = sum_{j != y} e^{z - m},
//            e = sum_{j != y} e^{z - m} z, sum z, the target's z when it lies in the
//            shard, and the shard's first-index argmax of the raw logits.
//   combine  per row over the shards (in ascending v0): lse, 1 - p_y, the loss,
//            log p_y and the entropy (labs-molt PR "Enable Liger layers": the
//            RL side needs action log-probabilities and entropy), the global
//            argmax, the counts and the reduced loss.
//   grad     the gradient of a shard in place, from lse and 1 - p_y, with the
//            reduction and upstream gradient given at this point.
//
// With one shard this is a forward / deferred-backward split; with several it
// is the local half of a vocabulary-parallel loss whose only exchange is the
// stats records (32 bytes per row and shard).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ce_device.h"
#include "lce_internal.h"

namespace lce {
namespace {

using dev::Elt;
using dev::kLog2e;
using dev::NT;
using dev::NWAVE;
using dev::u32x4;


// one thread's running statistics of a stretch of the row
struct Part {
    float m = -FLT_MAX;   // running max of z (finite start: no inf - inf)
    float s = 0.0f;       // sum over j != target of e^{z - m}
    float e = 0.0f;       // sum over j != target of e^{z - m} z
    float zs = 0.0f;      // sum of z
    float amv = -INFINITY;
    int am = 0x7fffffff;  // shard-local index of the first maximum of the raw logits
};

__device__ __forceinline__ void combine(Part &a, float m2, float s2, float e2) {
    const float M = fmaxf(a.m, m2);
    const float f1 = dev::exp2_fast((a.m - M) * kLog2e), f2 = dev::exp2_fast((m2 - M) * kLog2e);
    a.s = a.s * f1 + s2 * f2;
    a.e = a.e * f1 + e2 * f2;
    a.m = M;
}

template <int CTRL>
__device__ __forceinline__ void part_step(Part &p) {
    const float m2 = dev::dpp_f<CTRL>(p.m), s2 = dev::dpp_f<CTRL>(p.s), e2 = dev::dpp_f<CTRL>(p.e);
    const float z2 = dev::dpp_f<CTRL>(p.zs);
    combine(p, m2, s2, e2);
    p.zs += z2;
}
// the wave's (m, s, e, sum z), the same in every lane (each step combines the
// same two operands in both lanes)
__device__ __forceinline__ void wave_part(Part &p) {
    part_step<dev::kDppXor1>(p);
    part_step<dev::kDppXor2>(p);
    part_step<dev::kDppHalfMirror>(p);
    part_step<dev::kDppMirror>(p);
    Part r[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        r[q].m = dev::lane_f(p.m, 16 * q);
        r[q].s = dev::lane_f(p.s, 16 * q);
        r[q].e = dev::lane_f(p.e, 16 * q);
        r[q].zs = dev::lane_f(p.zs, 16 * q);
    }
    combine(r[0], r[1].m, r[1].s, r[1].e);
    r[0].zs += r[1].zs;
    combine(r[2], r[3].m, r[3].s, r[3].e);
    r[2].zs += r[3].zs;
    combine(r[0], r[2].m, r[2].s, r[2].e);
    r[0].zs += r[2].zs;
    p.m = r[0].m;
    p.s = r[0].s;
    p.e = r[0].e;
    p.zs = r[0].zs;
}

#ifndef LCE_STATS_THREADS
#define LCE_STATS_THREADS 256
#endif
#ifndef LCE_STATS_AHEAD
#define LCE_STATS_AHEAD 4
#endif
#ifndef LCE_GRAD_PER
#define LCE_GRAD_PER 4
#endif
constexpr int kStatsThreads = LCE_STATS_THREADS;      // four waves per row: several rows per CU
constexpr int kStatsWaves = kStatsThreads / 64;
constexpr int kStatsAhead = LCE_STATS_AHEAD;          // 16-byte vectors per batch; two batches in flight
constexpr int kGradPer = LCE_GRAD_PER;                // 16-byte vectors per thread of the gradient (shards < 8192 vectors)

template <bool BF16, bool SOFTCAP>
__global__ __launch_bounds__(kStatsThreads) void ce_stats_kernel(const void *logits, int64_t ld, int64_t Vs,
                                                                 int64_t v0, const int64_t *labels,
                                                                 int64_t ignore_index, float softcap, float *stats) {
    using EL = Elt<BF16>;
    constexpr int E = EL::E;
    constexpr int NTS = kStatsThreads;
    __shared__ float sh[5][kStatsWaves];
    __shared__ int sh_i[kStatsWaves];
    const int64_t row = blockIdx.x;
    const int tid = threadIdx.x;
    const int nvec = static_cast<int>(Vs / E);
    const int64_t y = labels[row];
    const int yl = (y != ignore_index && y >= v0 && y < v0 + Vs) ? static_cast<int>(y - v0) : -1;   // in shard
    const int yv = yl >= 0 ? yl / E : -1, ye = yl >= 0 ? yl % E : 0;
    const dev::Cap cap{SOFTCAP ? 2.0f * kLog2e / softcap : 0.0f, softcap};
    const __amdgpu_buffer_rsrc_t src = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char *>(static_cast<const char *>(logits)) + row * ld * EL::bytes, 0,
        static_cast<uint32_t>(nvec) * 16u, 0x00020000);

    Part p;
    float zy = 0.0f;
    // two batches of loads in flight: the next batch goes out before this one is used
    // (past the row, on the last pass too, the descriptor returns zeros without a memory access).
    // Default cache policy, not non-temporal: the shard may stay in the 256 MB Infinity Cache for
    // the gradient pass, which reads it again.
    u32x4 v[kStatsAhead];
#pragma unroll
    for (int u = 0; u < kStatsAhead; ++u)
        v[u] = __builtin_amdgcn_raw_buffer_load_b128(src, (u * NTS + tid) * 16, 0, 0);
    for (int base = 0; base < nvec; base += NTS * kStatsAhead) {
        u32x4 nx[kStatsAhead];
#pragma unroll
        for (int u = 0; u < kStatsAhead; ++u)
            nx[u] = __builtin_amdgcn_raw_buffer_load_b128(src, (base + (kStatsAhead + u) * NTS + tid) * 16, 0, 0);
#pragma unroll
        for (int u = 0; u < kStatsAhead; ++u) {
            const int vi = base + u * NTS + tid;
            if (vi >= nvec) continue;
            float x[E], z[E];
            float rmax = -FLT_MAX, xmax = -INFINITY;
#pragma unroll
            for (int k = 0; k < E; ++k) {
                x[k] = EL::get(v[u], k);
                z[k] = SOFTCAP ? cap.z_of_r(cap.r_of(x[k])) : x[k];
                if constexpr (SOFTCAP) rmax = fmaxf(rmax, z[k]);
                xmax = fmaxf(xmax, x[k]);
            }
            if constexpr (!SOFTCAP) rmax = fmaxf(xmax, -FLT_MAX);   // z = x: one max chain
            if (xmax > p.amv) {   // vectors come in index order per thread: keep the first
                int first = E - 1;
#pragma unroll
                for (int k = E - 2; k >= 0; --k)
                    if (x[k] == xmax) first = k;
                p.amv = xmax;
                p.am = vi * E + first;
            }
            // Every weight here carries the same rounding of mn * log2e (|mn| * 2^-24
            // relative), which cancels between s and e; the target's weight is formed
            // exactly in the combine, so the target stays out of both sums (inside e it would
            // leave an entropy error of |z_y| times that rounding).
            const float mn = fmaxf(p.m, rmax), mnL = mn * kLog2e;
            const float f = dev::exp2_fast(fmaf(p.m, kLog2e, -mnL));
            float ex[E], pe = 0.0f, zsum = 0.0f;
#pragma unroll
            for (int k = 0; k < E; ++k) {
                ex[k] = dev::exp2_fast(fmaf(z[k], kLog2e, -mnL));
                zsum += z[k];
            }
            if (vi == yv) {   // the target's vector: its element stays out of s and e
#pragma unroll
                for (int k = 0; k < E; ++k)
                    if (k == ye) {
                        zy = z[k];
                        ex[k] = 0.0f;
                    }
            }
#pragma unroll
            for (int k = 0; k < E; ++k) pe = fmaf(ex[k], z[k], pe);
            float ps = ex[0];
#pragma unroll
            for (int k = 1; k < E; ++k) ps += ex[k];
            p.zs += zsum;
            p.s = fmaf(p.s, f, ps);
            p.e = fmaf(p.e, f, pe);
            p.m = mn;
        }
#pragma unroll
        for (int u = 0; u < kStatsAhead; ++u) v[u] = nx[u];
    }
    // wave (DPP exchanges, then the four 16-lane rows in a fixed order), then workgroup
    wave_part(p);
    dev::wave_argmax_dpp(p.amv, p.am);
    const int w = tid >> 6;
    if ((tid & 63) == 0) {
        sh[0][w] = p.m;
        sh[1][w] = p.s;
        sh[2][w] = p.e;
        sh[3][w] = p.zs;
        sh[4][w] = p.amv;
        sh_i[w] = p.am;
    }
    __syncthreads();
    if (tid == 0) {
        Part t;
        t.m = sh[0][0];
        t.s = sh[1][0];
        t.e = sh[2][0];
        t.zs = sh[3][0];
        t.amv = sh[4][0];
        t.am = sh_i[0];
        for (int k = 1; k < kStatsWaves; ++k) {
            combine(t, sh[0][k], sh[1][k], sh[2][k]);
            t.zs += sh[3][k];
            dev::argmax_combine(t.amv, t.am, sh[4][k], sh_i[k]);
        }
        float *o = stats + row * 8;
        o[0] = t.m;
        o[1] = t.s;
        o[2] = t.e;
        o[3] = t.zs;
        o[4] = t.amv;
        o[5] = __int_as_float(static_cast<int>(v0 + t.am));   // global index (V < 2^31)
        if (yl < 0) {
            o[6] = 0.0f;
            o[7] = 0.0f;
        }
    }
    // the target's z, from the thread that read it
    if (yl >= 0 && tid == yv % NTS) {
        stats[row * 8 + 6] = zy;
        stats[row * 8 + 7] = 1.0f;
    }
}

// per row over the shards: outputs; n_correct by integer atomics (order-free)
__global__ __launch_bounds__(256) void ce_combine_kernel(const float *stats, int64_t shards, int64_t shard_stride,
                                                         int64_t row_stride, const int64_t *labels, int64_t n, int64_t V,
                                                         int64_t ignore_index, float eps, float *lse_out,
                                                         float *q_out, float *loss_tok, float *logp_out,
                                                         float *ent_out, int64_t *argmax_out, int64_t *counts) {
    const int64_t i = blockIdx.x * 256ll + threadIdx.x;
    if (i >= n) return;
    Part t;
    float zy = 0.0f;
    bool has = false;
    int64_t am = -1;
    // the next shard's record is loaded before this one is merged (the last pass
    // reloads its own record: an unconditional load of a valid address)
    const float4 *rec = reinterpret_cast<const float4 *>(stats + i * row_stride * 8);
    const int64_t step = shard_stride * 2;   // float4s per shard
    float4 a = rec[0], b = rec[1];
    for (int64_t k = 0; k < shards; ++k) {
        const int64_t kn = k + 1 < shards ? k + 1 : k;
        const float4 na = rec[kn * step], nb = rec[kn * step + 1];
        combine(t, a.x, a.y, a.z);
        t.zs += a.w;
        if (b.x > t.amv) {   // shards in ascending vocabulary order: ties keep the earlier
            t.amv = b.x;
            am = __float_as_int(b.y);
        }
        if (b.w != 0.0f) {
            zy = b.z;
            has = true;
        }
        a = na;
        b = nb;
    }
    const int64_t y = labels[i];
    const bool valid = y != ignore_index && y >= 0 && y < V;
    const float ey = has ? dev::exp2_fast((zy - t.m) * kLog2e) : 0.0f;
    const float S = t.s + ey;
    const float lse = t.m + logf(S);
    lse_out[i] = lse;
    if (q_out) q_out[i] = valid ? t.s / S : 0.0f;
    if (loss_tok) loss_tok[i] = valid ? lse - (1.0f - eps) * zy - eps / static_cast<float>(V) * t.zs : 0.0f;
    if (logp_out) logp_out[i] = valid ? zy - lse : 0.0f;
    if (ent_out) ent_out[i] = lse - fmaf(ey, zy, t.e) / S;   // -sum p log p = lse - sum p z
    if (argmax_out) argmax_out[i] = am;
    if (valid && am == y) __hip_atomic_fetch_add(reinterpret_cast<unsigned long long *>(counts + 1), 1ull,
                                                  __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One row's results from its records over at most a few shards: eight shards'
// records in flight at a time (clamped to the last shard), merged in ascending
// shard order.
struct RowOut {
    float lse, q, loss, logp, ent;
    int64_t am;
    bool valid;
};
__device__ __forceinline__ RowOut combine_row(const float *stats, int64_t shards, int64_t shard_stride,
                                              int64_t row_stride, int64_t i, int64_t y, int64_t V,
                                              int64_t ignore_index, float eps) {
    Part t;
    float zy = 0.0f;
    bool has = false;
    int64_t am = -1;
    const float4 *rec = reinterpret_cast<const float4 *>(stats + i * row_stride * 8);
    const int64_t step = shard_stride * 2;   // float4s per shard
    constexpr int kBatch = 8;
    for (int64_t k0 = 0; k0 < shards; k0 += kBatch) {
        float4 ra[kBatch], rb[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int64_t k = k0 + u < shards ? k0 + u : shards - 1;
            ra[u] = rec[k * step];
            rb[u] = rec[k * step + 1];
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            if (k0 + u >= shards) break;
            combine(t, ra[u].x, ra[u].y, ra[u].z);
            t.zs += ra[u].w;
            if (rb[u].x > t.amv) {   // shards in ascending vocabulary order: ties keep the earlier
                t.amv = rb[u].x;
                am = __float_as_int(rb[u].y);
            }
            if (rb[u].w != 0.0f) {
                zy = rb[u].z;
                has = true;
            }
        }
    }
    RowOut o;
    o.valid = y != ignore_index && y >= 0 && y < V;
    const float ey = has ? dev::exp2_fast((zy - t.m) * kLog2e) : 0.0f;
    const float S = t.s + ey;
    o.lse = t.m + logf(S);
    o.q = o.valid ? t.s / S : 0.0f;
    o.loss = o.valid ? o.lse - (1.0f - eps) * zy - eps / static_cast<float>(V) * t.zs : 0.0f;
    o.logp = o.valid ? zy - o.lse : 0.0f;
    o.ent = o.lse - fmaf(ey, zy, t.e) / S;   // -sum p log p = lse - sum p z
    o.am = am;
    return o;
}

// reduction 1 (mean over valid labels), 2 (sum), else 0
__device__ __forceinline__ float reduce_loss(double tot, long long n_valid, int reduction) {
    if (reduction == 1) return n_valid > 0 ? static_cast<float>(tot / static_cast<double>(n_valid)) : 0.0f;
    if (reduction == 2) return static_cast<float>(tot);
    return 0.0f;
}

// The whole combine in one workgroup, for up to kCombineOneMaxRows rows of a
// few shards: row outputs, label counts, n_correct and the reduced loss, with
// no atomics and no second launch.  Thread t takes rows t, t + 1024, ...; the
// counts and the fp64 loss sum fold over the threads in a fixed order.
constexpr int kCombineOneThreads = 1024;
constexpr int64_t kCombineOneMaxRows = 16384;
__global__ __launch_bounds__(kCombineOneThreads) void ce_combine_one_kernel(
    const float *stats, int64_t shards, int64_t shard_stride, int64_t row_stride, const int64_t *labels, int64_t n,
    int64_t V, int64_t ignore_index, float eps, int reduction, float *lse_out, float *q_out, float *loss_tok,
    float *loss_out, float *logp_out, float *ent_out, int64_t *argmax_out, int64_t *counts) {
    constexpr int NW = kCombineOneThreads / 64;
    __shared__ double sh_d[NW];
    __shared__ long long sh_c[3][NW];
    const int tid = threadIdx.x;
    double acc = 0.0;
    long long nv = 0, nc = 0, nb = 0;
    for (int64_t i = tid; i < n; i += kCombineOneThreads) {
        const int64_t y = labels[i];
        const RowOut o = combine_row(stats, shards, shard_stride, row_stride, i, y, V, ignore_index, eps);
        if (y != ignore_index) {
            if (o.valid) ++nv;
            else ++nb;
        }
        lse_out[i] = o.lse;
        if (q_out) q_out[i] = o.q;
        if (loss_tok) loss_tok[i] = o.loss;
        if (logp_out) logp_out[i] = o.logp;
        if (ent_out) ent_out[i] = o.ent;
        if (argmax_out) argmax_out[i] = o.am;
        if (o.valid && o.am == y) ++nc;
        acc += static_cast<double>(o.loss);
    }
    acc = dev::wave_sum_d(acc);
    nv = dev::wave_sum_ll(nv);
    nc = dev::wave_sum_ll(nc);
    nb = dev::wave_sum_ll(nb);
    if ((tid & 63) == 0) {
        sh_d[tid >> 6] = acc;
        sh_c[0][tid >> 6] = nv;
        sh_c[1][tid >> 6] = nc;
        sh_c[2][tid >> 6] = nb;
    }
    __syncthreads();
    if (tid == 0) {
        double tot = 0.0;
        long long c[3] = {0, 0, 0};
        for (int w = 0; w < NW; ++w) {
            tot += sh_d[w];
            for (int j = 0; j < 3; ++j) c[j] += sh_c[j][w];
        }
        counts[0] = c[0];
        counts[1] = c[1];
        counts[2] = c[2];
        if (loss_out) *loss_out = reduce_loss(tot, c[0], reduction);
    }
}

// The same over many workgroups, one row per thread, for more rows than one
// workgroup covers in a pass (it needs argmax_out, and loss_tok when loss_out is
// asked for).  The workgroups count their completions in counts[1] (a tagged
// word, so whatever it held before does not matter; the call overwrites it with
// n_correct at the end).  The last workgroup to finish counts the labels,
// compares the stored argmax with them for n_correct, and folds the per-token
// losses in a fixed order, so the result does not depend on which workgroup is
// last.  What it reads back (loss_tok, argmax_out) is stored at system scope
// and acknowledged before the count is drawn, so it reads them past its own L2.
#ifndef LCE_COMBINE_PAR_THREADS
#define LCE_COMBINE_PAR_THREADS 256
#endif
constexpr int kCombineParThreads = LCE_COMBINE_PAR_THREADS;
constexpr int kCombineParFold = 8;   // rows per thread in flight in the fold
__global__ __launch_bounds__(kCombineParThreads) void ce_combine_par_kernel(
    const float *stats, int64_t shards, int64_t shard_stride, int64_t row_stride, const int64_t *labels, int64_t n,
    int64_t V, int64_t ignore_index, float eps, int reduction, float *lse_out, float *q_out, float *loss_tok,
    float *loss_out, float *logp_out, float *ent_out, int64_t *argmax_out, int64_t *counts) {
    constexpr int NTH = kCombineParThreads;
    constexpr int NW = NTH / 64;
    __shared__ double sh_d[NW];
    __shared__ long long sh_c[3][NW];
    __shared__ int sh_last;
    const int tid = threadIdx.x;
    const unsigned tag = dev::launch_tag();
    unsigned long long *ticket = reinterpret_cast<unsigned long long *>(counts + 1);
    if (tid == 0) dev::tagged_claim(ticket, tag);
    const int64_t i = static_cast<int64_t>(blockIdx.x) * NTH + tid;
    if (i < n) {
        const int64_t y = labels[i];
        const RowOut o = combine_row(stats, shards, shard_stride, row_stride, i, y, V, ignore_index, eps);
        lse_out[i] = o.lse;
        if (q_out) q_out[i] = o.q;
        if (logp_out) logp_out[i] = o.logp;
        if (ent_out) ent_out[i] = o.ent;
        if (loss_tok) dev::store_through(loss_tok + i, o.loss);
        __hip_atomic_store(reinterpret_cast<unsigned long long *>(argmax_out + i),
                           static_cast<unsigned long long>(o.am), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0) sh_last = dev::tagged_draw(ticket, tag) == gridDim.x - 1u;
    __syncthreads();
    if (!sh_last) return;
    // fixed order: thread t takes rows t, t + NTH, ... (kCombineParFold in flight), then the
    // waves in order
    double acc = 0.0;
    long long nv = 0, nc = 0, nb = 0;
    for (int64_t r0 = 0; r0 < n; r0 += kCombineParFold * NTH) {
        int64_t yv[kCombineParFold];
        unsigned long long av[kCombineParFold];
        float lv[kCombineParFold];
#pragma unroll
        for (int u = 0; u < kCombineParFold; ++u) {
            int64_t r = r0 + u * NTH + tid;
            r = r < n ? r : n - 1;
            yv[u] = labels[r];
            av[u] = __hip_atomic_load(reinterpret_cast<unsigned long long *>(argmax_out + r), __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_SYSTEM);
            lv[u] = loss_tok ? __uint_as_float(__hip_atomic_load(reinterpret_cast<unsigned *>(loss_tok) + r,
                                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM))
                             : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < kCombineParFold; ++u) {
            if (r0 + u * NTH + tid >= n) break;
            const int64_t y = yv[u];
            if (y == ignore_index) continue;
            if (y >= 0 && y < V) {
                ++nv;
                if (static_cast<int64_t>(av[u]) == y) ++nc;
            } else {
                ++nb;
            }
            acc += static_cast<double>(lv[u]);
        }
    }
    acc = dev::wave_sum_d(acc);
    nv = dev::wave_sum_ll(nv);
    nc = dev::wave_sum_ll(nc);
    nb = dev::wave_sum_ll(nb);
    if ((tid & 63) == 0) {
        sh_d[tid >> 6] = acc;
        sh_c[0][tid >> 6] = nv;
        sh_c[1][tid >> 6] = nc;
        sh_c[2][tid >> 6] = nb;
    }
    __syncthreads();
    if (tid == 0) {
        double tot = 0.0;
        long long c[3] = {0, 0, 0};
        for (int w = 0; w < NW; ++w) {
            tot += sh_d[w];
            for (int j = 0; j < 3; ++j) c[j] += sh_c[j][w];
        }
        counts[0] = c[0];
        counts[2] = c[2];
        if (loss_out) *loss_out = reduce_loss(tot, c[0], reduction);
        counts[1] = c[1];   // replaces the completion count
    }
}

// Many shards per row (one per 256 columns in the tile-resident fused linear
// path): one wave per row, each lane merges every 64th shard in ascending
// order, then a butterfly merges the lanes (argmax ties to the smaller index).
__global__ __launch_bounds__(256) void ce_combine_wide_kernel(const float *stats, int64_t shards,
                                                              int64_t shard_stride, int64_t row_stride,
                                                              const int64_t *labels, int64_t n, int64_t V,
                                                              int64_t ignore_index, float eps, float *lse_out,
                                                              float *q_out, float *loss_tok, float *logp_out,
                                                              float *ent_out, int64_t *argmax_out, int64_t *counts) {
    const int64_t i = blockIdx.x * 4ll + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (i >= n) return;   // uniform over the wave
    Part t;
    float zy = 0.0f, has = 0.0f;
    for (int64_t k = lane; k < shards; k += 64) {
        const float4 *r = reinterpret_cast<const float4 *>(stats + (k * shard_stride + i * row_stride) * 8);
        const float4 a = r[0], b = r[1];
        combine(t, a.x, a.y, a.z);
        t.zs += a.w;
        if (b.x > t.amv) {   // this lane's shards ascend: ties keep the earlier
            t.amv = b.x;
            t.am = __float_as_int(b.y);
        }
        if (b.w != 0.0f) {
            zy = b.z;
            has = 1.0f;
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        combine(t, __shfl_xor(t.m, o, 64), __shfl_xor(t.s, o, 64), __shfl_xor(t.e, o, 64));
        t.zs += __shfl_xor(t.zs, o, 64);
        dev::argmax_combine(t.amv, t.am, __shfl_xor(t.amv, o, 64), __shfl_xor(t.am, o, 64));
        zy += __shfl_xor(zy, o, 64);   // at most one lane holds the target
        has += __shfl_xor(has, o, 64);
    }
    if (lane != 0) return;
    const int64_t y = labels[i];
    const bool valid = y != ignore_index && y >= 0 && y < V;
    const float ey = has != 0.0f ? dev::exp2_fast((zy - t.m) * kLog2e) : 0.0f;
    const float S = t.s + ey;
    const float lse = t.m + logf(S);
    const int64_t am = t.am;
    lse_out[i] = lse;
    if (q_out) q_out[i] = valid ? t.s / S : 0.0f;
    if (loss_tok) loss_tok[i] = valid ? lse - (1.0f - eps) * zy - eps / static_cast<float>(V) * t.zs : 0.0f;
    if (logp_out) logp_out[i] = valid ? zy - lse : 0.0f;
    if (ent_out) ent_out[i] = lse - fmaf(ey, zy, t.e) / S;
    if (argmax_out) argmax_out[i] = am;
    if (valid && am == y) __hip_atomic_fetch_add(reinterpret_cast<unsigned long long *>(counts + 1), 1ull,
                                                  __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <bool BF16, bool SOFTCAP, bool SMOOTH, int PER>   // PER: 16-byte vectors per thread
__global__ __launch_bounds__(256) void ce_grad_kernel(void *logits, int64_t ld, int64_t Vs, int64_t v0, int64_t V,
                                                      const int64_t *labels, int64_t ignore_index, float eps,
                                                      float softcap, int reduction, const float *grad_out,
                                                      const float *lse, const float *q, const int64_t *counts,
                                                      int blocks_per_row) {
    using EL = Elt<BF16>;
    constexpr int E = EL::E;
    const int64_t row = blockIdx.x / blocks_per_row;
    const int part = blockIdx.x % blocks_per_row;
    const int nvec = static_cast<int>(Vs / E);
    const int64_t y = labels[row];
    const bool valid = y != ignore_index && y >= 0 && y < V;
    const int64_t nv = counts[0];
    const float g = reduction == 0 ? (grad_out ? grad_out[row] : 1.0f) : (grad_out ? grad_out[0] : 1.0f);
    const float scale = !valid ? 0.0f : (reduction == 1 ? (nv > 0 ? g / static_cast<float>(nv) : 0.0f) : g);
    const int64_t yl = (valid && y >= v0 && y < v0 + Vs) ? y - v0 : -1;
    const dev::Cap cap{SOFTCAP ? 2.0f * kLog2e / softcap : 0.0f, softcap};
    char *rowp = static_cast<char *>(logits) + row * ld * EL::bytes;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(rowp, 0, static_cast<uint32_t>(nvec) * 16u,
                                                                        0x00020000);
    const int v_first = part * 256 * PER + threadIdx.x;
    if (scale == 0.0f) {
        // ignored rows (and a zero upstream gradient): zeros, nothing to read
#pragma unroll
        for (int u = 0; u < PER; ++u)
            __builtin_amdgcn_raw_buffer_store_b128((u32x4){0u, 0u, 0u, 0u}, rs, (v_first + u * 256) * 16, 0, 2);
        return;
    }
    const float ascale = fabsf(scale);
    const bool negate = scale < 0.0f;
    const float lseL = lse[row] * kLog2e - log2f(ascale);
    const float epsV = SMOOTH ? eps / static_cast<float>(V) * ascale : 0.0f;
    const float capk = -2.0f * softcap * kLog2e, capb2 = (softcap - lse[row]) * kLog2e + log2f(ascale);
    u32x4 v[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) v[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, (v_first + u * 256) * 16, 0, 2);
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int vi = v_first + u * 256;
        float gv[E];
#pragma unroll
        for (int k = 0; k < E; ++k) {
            const float x = EL::get(v[u], k);
            if constexpr (SOFTCAP) {
                float r, q;
                cap.r_q(x, r, q);
                const float pp = dev::exp2_fast(fmaf(r, capk, capb2));   // |s| p_j
                gv[k] = (SMOOTH ? pp - epsV : pp) * dev::Cap::chain(r, q);
            } else {
                const float pp = dev::exp2_fast(fmaf(x, kLog2e, -lseL));
                gv[k] = SMOOTH ? pp - epsV : pp;
            }
        }
        if (yl >= 0 && yl / E == vi) {
            // the target: s (p_y - (1 - eps) - eps / V) with p_y - 1 = -(1 - p_y)
            const int k = static_cast<int>(yl % E);
            float gy = ascale * (eps - q[row] - (SMOOTH ? eps / static_cast<float>(V) : 0.0f));
            if constexpr (SOFTCAP) {
                float ry, qy;
                cap.r_q(EL::get(v[u], k), ry, qy);
                gy *= dev::Cap::chain(ry, qy);
            }
#pragma unroll
            for (int kk = 0; kk < E; ++kk)
                if (kk == k) gv[kk] = gy;
        }
        if (negate) {
#pragma unroll
            for (int k = 0; k < E; ++k) gv[k] = -gv[k];
        }
        // lanes past the row are outside the descriptor: dropped
        __builtin_amdgcn_raw_buffer_store_b128(EL::pack(gv), rs, vi * 16, 0, 2);
    }
}

}  // namespace

hipError_t launch_ce_stats(const void *logits, int64_t ld, bool is_bf16, const int64_t *labels, int64_t n,
                           int64_t Vs, int64_t v0, int64_t ignore_index, float softcap, float *stats,
                           hipStream_t st) {
    if (n == 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>(n)), block(kStatsThreads);
    const bool sc = softcap > 0.0f;
    if (is_bf16) {
        if (sc) hipLaunchKernelGGL((ce_stats_kernel<true, true>), grid, block, 0, st, logits, ld, Vs, v0, labels, ignore_index, softcap, stats);
        else hipLaunchKernelGGL((ce_stats_kernel<true, false>), grid, block, 0, st, logits, ld, Vs, v0, labels, ignore_index, softcap, stats);
    } else {
        if (sc) hipLaunchKernelGGL((ce_stats_kernel<false, true>), grid, block, 0, st, logits, ld, Vs, v0, labels, ignore_index, softcap, stats);
        else hipLaunchKernelGGL((ce_stats_kernel<false, false>), grid, block, 0, st, logits, ld, Vs, v0, labels, ignore_index, softcap, stats);
    }
    return hipGetLastError();
}

hipError_t launch_ce_combine(const float *stats, int64_t shards, int64_t shard_stride, int64_t row_stride,
                             const int64_t *labels, int64_t n, int64_t V, int64_t ignore_index, float eps, int reduction, float *lse,
                             float *q, float *loss_tok, float *loss_out, float *logp, float *ent,
                             int64_t *argmax_out, int64_t *counts, hipStream_t st) {
    hipError_t e;
    // many workgroups for several shards beyond one pass of the one-workgroup form (with one
    // shard, whose rows are cheap to merge, its two passes cost less than the completion count
    // and the fold), and for every shape past that form's row limit
    if (shards <= 16 && argmax_out && (n > kCombineOneMaxRows || (shards > 1 && n > kCombineOneThreads))) {
        const dim3 grid(static_cast<unsigned>((n + kCombineParThreads - 1) / kCombineParThreads));
        hipLaunchKernelGGL(ce_combine_par_kernel, grid, dim3(kCombineParThreads), 0, st, stats, shards, shard_stride,
                           row_stride, labels, n, V, ignore_index, eps, reduction, lse, q, loss_tok, loss_out, logp,
                           ent, argmax_out, counts);
        return hipGetLastError();
    }
    if (shards <= 16 && n <= kCombineOneMaxRows) {
        // one launch does everything (n == 0 included: counts and loss_out become 0)
        hipLaunchKernelGGL(ce_combine_one_kernel, dim3(1), dim3(kCombineOneThreads), 0, st, stats, shards,
                           shard_stride, row_stride, labels, n, V, ignore_index, eps, reduction, lse, q, loss_tok,
                           loss_out, logp, ent, argmax_out, counts);
        return hipGetLastError();
    }
    // counts {n_valid, 0, n_bad}; n_correct is added below
    if ((e = launch_ce_count(labels, n, V, ignore_index, counts, nullptr, loss_out, st)) != hipSuccess) return e;
    if (n > 0 && shards > 16) {
        const dim3 grid(static_cast<unsigned>((n + 3) / 4)), block(256);
        hipLaunchKernelGGL(ce_combine_wide_kernel, grid, block, 0, st, stats, shards, shard_stride, row_stride, labels,
                           n, V, ignore_index, eps, lse, q, loss_tok, logp, ent, argmax_out, counts);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    } else if (n > 0) {
        const dim3 grid(static_cast<unsigned>((n + 255) / 256)), block(256);
        hipLaunchKernelGGL(ce_combine_kernel, grid, block, 0, st, stats, shards, shard_stride, row_stride, labels, n,
                           V, ignore_index, eps, lse, q, loss_tok, logp, ent, argmax_out, counts);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (loss_out) return launch_loss_fold(loss_tok, n, counts, reduction, loss_out, st);
    return hipSuccess;
}

hipError_t launch_ce_grad(void *logits, int64_t ld, bool is_bf16, const int64_t *labels, int64_t n, int64_t Vs,
                          int64_t v0, int64_t V, int64_t ignore_index, float eps, float softcap, int reduction,
                          const float *grad_out, const float *lse, const float *q, const int64_t *counts,
                          hipStream_t st) {
    if (n == 0) return hipSuccess;
    const int E = is_bf16 ? 8 : 4;
    const int64_t nvec = Vs / E;
    // eight vectors per thread on long shards (fewer, larger workgroups: measured faster at 16384
    // vectors, slower at 2048), else four
    const bool wide = nvec >= 8192;
    const int per = wide ? 8 : kGradPer;
    const int bpr = static_cast<int>((nvec + 256 * per - 1) / (256 * per));
    const dim3 grid(static_cast<unsigned>(n * bpr)), block(256);
    const bool sc = softcap > 0.0f, sm = eps != 0.0f;
#define LCE_GRAD(B, S, M)                                                                                          \
    do {                                                                                                           \
        if (wide)                                                                                                  \
            hipLaunchKernelGGL((ce_grad_kernel<B, S, M, 8>), grid, block, 0, st, logits, ld, Vs, v0, V, labels,    \
                               ignore_index, eps, softcap, reduction, grad_out, lse, q, counts, bpr);              \
        else                                                                                                       \
            hipLaunchKernelGGL((ce_grad_kernel<B, S, M, kGradPer>), grid, block, 0, st, logits, ld, Vs, v0, V,      \
                               labels,                                                                              \
                               ignore_index, eps, softcap, reduction, grad_out, lse, q, counts, bpr);              \
    } while (0)
    if (is_bf16) {
        if (sc) { if (sm) LCE_GRAD(true, true, true); else LCE_GRAD(true, true, false); }
        else { if (sm) LCE_GRAD(true, false, true); else LCE_GRAD(true, false, false); }
    } else {
        if (sc) { if (sm) LCE_GRAD(false, true, true); else LCE_GRAD(false, true, false); }
        else { if (sm) LCE_GRAD(false, false, true); else LCE_GRAD(false, false, false); }
    }
#undef LCE_GRAD
    return hipGetLastError();
}

}  // namespace lce
