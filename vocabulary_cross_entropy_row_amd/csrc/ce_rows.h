// Persistent, software-pipelined cross-entropy row kernel (gfx950).
//
// Per row i, label y, eps = label smoothing, T = softcap:
//   z = T > 0 ? T tanh(x / T) : x
//   loss_i = LSE(z) - (1 - eps) z_y - (eps / V) sum_j z_j
//   dx_ij  = s_i (softmax(z)_j - (1 - eps)[j == y] - eps / V) dz_j / dx_j
// (Liger-Kernel PR "Add Megatron-LM cross-entropy integration", Summary and
// Test setup; Megatron-LM PR "Add opt-in Liger vocab-parallel cross entropy",
// "What does this PR do?"; Liger-Kernel PR "Add Liger Kernel support for Muse
// Glimmer", Details/Softcap.)
//
// Layout of the work: one 1024-thread workgroup per CU walks rows
// blockIdx.x, blockIdx.x + G, ...  A row is split into K rounds of 1024
// 16-byte vectors; thread t owns vector (k * 1024 + t) of every round.  The
// first KL rounds live in thread-private LDS slots filled by direct
// buffer->LDS loads, the remaining KR rounds in VGPRs, so the row is read
// from HBM once.  Two passes run over the resident row:
//   pass A, round by round as the data arrives: an online softmax (each
//           thread keeps a running max m and the sum of exp(z - m) over its
//           elements, rescaled when m grows), the argmax and sum z when asked;
//   pass B, once the row's statistics are combined: the gradient.
// Pass B handles the LDS rounds first; once they are stored, the LDS rounds of
// the workgroup's next row are requested, and they stream in while pass B
// finishes the register rounds.  Then the register rounds of the next row go
// out, and pass A of that row starts on its (by then resident) LDS rounds.
// So the HBM traffic of one row overlaps the arithmetic of the previous one.
//
// Rows are handed out dynamically: a workgroup starts on row blockIdx.x and
// then draws row numbers from a counter in the workspace, one row ahead of
// need, so CUs that stream faster (the XCDs differ by a few percent) take more
// rows and all workgroups finish within about one row of each other.
//
// The workgroups count the labels themselves (the mean scale needs n_valid
// before any gradient is written).  The last workgroup to finish sums the
// per-token losses in row order and the per-workgroup n_correct counts, so
// every reduction is deterministic whichever workgroup took which row.
#pragma once

#include <type_traits>

#include "ce_device.h"

namespace lce {
namespace dev {

// Ignored rows one draw may step over; past that the ignored row is processed
// (with scale 0) instead of drawing again.
constexpr int kSkipMax = 16;
// Rows per chunk of the end-of-call pass that zeroes ignored rows.
constexpr int kZeroChunk = 64;


// Row draws and the final fold's operands go through system-scope atomics:
// they are performed at, or written through to, memory, so workgroups on
// different XCDs (each with its own L2) see each other's values without a
// cache-wide writeback or invalidate.


// UA (unaligned rows): a row need not start on a 16-byte boundary (odd V, ld not
// a multiple of the vector, or an unaligned base).  The row is then read
// through the 16-byte aligned window that holds it: its first vector may start
// with elements of the row before and its last may end with elements of the
// row after.  Those elements are masked in pass A, and the lane holding such a
// boundary vector stores only the row's own elements of it, one at a time
// (its 16-byte store is dropped by an out-of-range offset), so the rows around
// are never written.
template <bool BF16, int KR, int KL, bool SOFTCAP, bool ARGMAX, bool SMOOTH, bool UA>
__global__ __launch_bounds__(NT) void ce_rows_kernel(CEArgs a) {
    using EL = Elt<BF16>;
    constexpr int E = EL::E;
    constexpr int K = KR + KL;
    constexpr int KRV = KR > 0 ? KR : 1;
    __shared__ u32x4 lds_rows[KL > 0 ? KL * NT : 1];
    // per-row combine slots, double-buffered by row parity: a wave still
    // reading row r's slots is at most one barrier behind a wave writing row
    // r+1's, never two
    __shared__ float sh_m[2][NWAVE], sh_s[2][NWAVE], sh_z[2][NWAVE], sh_zs[2][NWAVE];
    __shared__ int sh_i[2][NWAVE];
    __shared__ long long sh_c[2][NWAVE];   // label count partials (valid, bad) per wave
    __shared__ long long sh_k[NWAVE];      // n_correct partials of the final fold
    __shared__ double sh_d[NWAVE];
    __shared__ float sh_xy[2];
    __shared__ int sh_flag;
    // the schedule, published by thread 0 at each row's combine barrier
    __shared__ int64_t sh_next[2];
    __shared__ unsigned long long sh_ign[2];   // ignored rows of a zeroing chunk
    __shared__ unsigned sh_chunk[2];

    const int tid = threadIdx.x;
    const int wave_base = tid & ~63;
    const int nvec = static_cast<int>(a.V / E);
    const int G = gridDim.x;
    const int64_t n = a.n;
    const float eps = a.eps;
    const float invV = 1.0f / static_cast<float>(a.V);
    const Cap cap{SOFTCAP ? 2.0f * kLog2e / a.softcap : 0.0f, a.softcap};
    const float capk = -2.0f * a.softcap * kLog2e;   // d(z log2 e)/dr under the softcap
    const u32x4 zero4 = {0u, 0u, 0u, 0u};
    // Labels and the upstream gradient are read-only for the kernel's lifetime:
    // read them through the constant address space, i.e. with scalar loads,
    // which wait on their own counter instead of on the row's vector loads.
    typedef const __attribute__((address_space(4))) int64_t *clabels_t;
    typedef const __attribute__((address_space(4))) float *cfloat_t;
    const clabels_t lab = (clabels_t)a.labels;
    const cfloat_t gout = (cfloat_t)a.grad_out;


    auto valid_label = [&](int64_t y) { return y != a.ignore_index && y >= 0 && y < a.V; };

    // Row memory goes through buffer instructions: the row base sits in a
    // uniform descriptor (SGPRs), every round shares one VGPR offset
    // (tid * 16) plus a scalar round offset, and the descriptor's range check
    // (num_records = the row's V * b bytes) drops the lanes of a partial last
    // round, so loads and stores need no exec masking.  When there is no row
    // to prefetch the descriptor is empty (num_records = 0): loads through it
    // return zeros without touching memory.  Reloading unconditionally lets
    // each register round die right after its last use.
    const uint32_t row_bytes = static_cast<uint32_t>(nvec) * 16u;
    const int Vi = static_cast<int>(a.V);
    // unaligned rows: the elements of the row before in row r's first vector,
    // and the number of vectors of its window
    auto row_off = [&](int64_t r) -> int {
        if constexpr (!UA) return 0;
        else
            return static_cast<int>((reinterpret_cast<uintptr_t>(a.logits) +
                                     static_cast<uintptr_t>(r * a.ld * EL::bytes)) & 15u) / EL::bytes;
    };
    auto row_nv = [&](int off) -> int { return UA ? (off + Vi + E - 1) / E : nvec; };
    auto row_rsrc = [&](int64_t r, bool live) {
        if constexpr (UA) {
            const int off = live ? row_off(r) : 0;
            return __builtin_amdgcn_make_buffer_rsrc(
                static_cast<char *>(a.logits) + (live ? r * a.ld * EL::bytes - off * EL::bytes : 0), 0,
                live ? static_cast<uint32_t>(row_nv(off)) * 16u : 0u, kBufferWord3);
        } else {
            return __builtin_amdgcn_make_buffer_rsrc(static_cast<char *>(a.logits) + (live ? r : 0) * a.ld * EL::bytes,
                                                     0, live ? row_bytes : 0u, kBufferWord3);
        }
    };
    // the boundary vector of an unaligned row's window that holds elements of
    // another row (idx: its vector index, off / nv: the window's geometry)
    auto boundary = [&](int idx, int off, int nv) {
        return (idx == 0 && off > 0) || (idx == nv - 1 && (off + Vi) % E != 0);
    };
    const int voff = tid * 16;

    // rounds [0, KL) in LDS, [KL, K) in registers
    u32x4 v[KRV];
    auto issue_round = [&](int k, __amdgpu_buffer_rsrc_t src) {
        if (k >= KL) {
            v[k >= KL ? k - KL : 0] = __builtin_amdgcn_raw_buffer_load_b128(src, voff, k * NT * 16, kNonTemporal);
        } else {
            // 16 bytes per lane, written to LDS at (wave-uniform base) + lane * 16
            typedef __attribute__((address_space(3))) void *lptr;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (lptr)(&lds_rows[k * NT + wave_base]), 16, voff,
                                                     k * NT * 16, 0, kNonTemporal);
        }
    };
    // stores of a partial last round need no guard: lanes past the row are
    // outside the descriptor and dropped.  Every wave therefore issues the
    // same memory operations, which the LDS waits below count on.
    // The round offset rides in the VGPR offset, not in soffset: a 16-byte
    // store's data registers can still be read after the store has issued,
    // and the compiler only keeps the next VALU writes of those registers
    // back when soffset is not a register.  With the offset in an SGPR, lanes
    // 12-15 of each 16-lane group have stored what the next instruction wrote.
    // (The add is formed at each store: hoisted, every round would hold its
    // own offset register.)
    auto store_round = [&](int k, __amdgpu_buffer_rsrc_t dst, u32x4 val, bool drop = false) {
        int vo = drop ? 0x40000000 : voff;   // past any descriptor's range: the store is dropped
        asm volatile("" : "+v"(vo));
        __builtin_amdgcn_raw_buffer_store_b128(val, dst, vo + k * NT * 16, 0, kNonTemporal);
    };
    // a boundary vector's own elements, one store each, taken from the packed
    // vector (element offsets within the window; positions outside the row are
    // skipped)
    // (the first element's offset is formed here, opaque to the optimiser:
    // hoisted, every round would keep its own offsets in registers)
    auto store_elems = [&](__amdgpu_buffer_rsrc_t dst, int idx, int off, const u32x4 &pk) {
        int p0 = idx * E - off;   // row position of element 0
        asm volatile("" : "+v"(p0));
#pragma unroll
        for (int e = 0; e < E; ++e) {
            if (p0 + e >= 0 && p0 + e < Vi) {
                const uint32_t w = e * EL::bytes / 4 == 0 ? pk.x : e * EL::bytes / 4 == 1 ? pk.y
                                 : e * EL::bytes / 4 == 2 ? pk.z : pk.w;
                if constexpr (BF16)
                    __builtin_amdgcn_raw_buffer_store_b16(static_cast<unsigned short>(w >> (16 * (e & 1))), dst,
                                                          (p0 + off + e) * 2, 0, kNonTemporal);
                else
                    __builtin_amdgcn_raw_buffer_store_b32(w, dst, (p0 + off + e) * 4, 0, kNonTemporal);
            }
        }
    };
    // a round of the resident row as a 16-byte vector
    auto round_vec = [&](int k) -> u32x4 { return k >= KL ? v[k >= KL ? k - KL : 0] : lds_rows[k * NT + tid]; };

    // zero gradient and loss of an ignored row: stores only
    auto zero_row = [&](int64_t r) {
        const __amdgpu_buffer_rsrc_t rz = row_rsrc(r, true);
        const int off = row_off(r), nv = row_nv(off);
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const bool bnd = UA && boundary(k * NT + tid, off, nv);
            store_round(k, rz, zero4, bnd);
            if constexpr (UA) {
                if (bnd) store_elems(rz, k * NT + tid, off, zero4);
            }
        }
        if (tid == 0) store_through(a.loss_tok + r, 0.0f);
    };

    // The mean scale needs every label counted before any gradient is written.
    // The first labels are requested ahead of the first row, so counting them
    // does not wait behind the row's loads.
    const int64_t yc0 = tid < a.count_n ? a.count_labels[tid] : a.ignore_index;
    const int64_t yc1 = tid + NT < a.count_n ? a.count_labels[tid + NT] : a.ignore_index;
    __builtin_amdgcn_sched_barrier(0);
    // the first row is this workgroup's own (the grid never exceeds n); an
    // ignored one is carried through with scale 0
    int64_t row = blockIdx.x;
    // thread 0's draw of the row after the next one: requested behind the LDS
    // rounds of a row, so it has landed when they have (resolved when used)
    const unsigned tag = launch_tag();
    unsigned long long draw = 0;
    bool drawn = false;
    {
        const __amdgpu_buffer_rsrc_t src = row_rsrc(row, row < n);
#pragma unroll
        for (int k = 0; k < K; ++k) {
            if (k == KL && tid == 0 && G < n) {
                tagged_claim(ws_rows(a.workspace), tag);
                draw = tagged_inc(ws_rows(a.workspace));
                drawn = true;
            }
            issue_round(k, src);
            __builtin_amdgcn_sched_barrier(0);   // issue in the order pass A consumes
        }
        // KR stores through an empty descriptor (dropped without touching memory):
        // every row's LDS rounds then have the same 2 KR memory operations issued
        // behind them, the first row's included, so one wait serves all rows
        const __amdgpu_buffer_rsrc_t none = row_rsrc(0, false);
#pragma unroll
        for (int k = KL; k < K; ++k) store_round(k, none, zero4);
    }

    count_labels_publish(a, sh_c, yc0, yc1);
    __syncthreads();
    const float g_all = (a.reduction != 0 && gout) ? gout[0] : 1.0f;
    float red_scale = g_all;
    {
        // only the float scale stays live through the row loop; the fold at the
        // end reads the counts again
        long long nv0, nb0;
        count_labels_read(sh_c, nv0, nb0);
        if (a.reduction == 1) red_scale = nv0 > 0 ? g_all / static_cast<float>(nv0) : 0.0f;
    }

    long long correct = 0;

    int pb = 0;   // parity of the row iteration (selects the combine slots)
    for (int64_t nxt; row < n; row = nxt, pb ^= 1) {
        const __amdgpu_buffer_rsrc_t rp = row_rsrc(row, true);
        const int64_t y64 = lab[row];
        const bool valid = valid_label(y64);     // always true unless ARGMAX
        const int y = valid ? static_cast<int>(y64) : 0;
        // an ignored row on the argmax path is carried through with scale 0, so
        // its gradient comes out as zeros
        const float scale = !valid ? 0.0f : (a.reduction == 0 ? (gout ? gout[row] : 1.0f) : red_scale);

        // the window's geometry (unaligned rows: elements of the row before
        // in the first vector, vectors in all, the round of the last one)
        const int off = row_off(row);
        const int nv = row_nv(off);
        const int k_last = (nv - 1) / NT;
        // where the target element lives: round ky, thread ty, element ey
        const int vy = (y + off) / E, ey = (y + off) % E, ky = vy / NT, ty = vy % NT;
        const bool owner = tid == ty;

        // ---- pass A: online softmax statistics, argmax, sum z; the target
        // element is kept out of the sum (1 - p_y is then formed without
        // cancellation) and its raw value is published through LDS
        float m = -FLT_MAX;      // running max of z (finite start: no inf - inf)
        float s = 0.0f;          // sum over this thread's elements j != y of exp(z_j - m)
        float zs = 0.0f;         // sum of z (label smoothing)
        float amv = -INFINITY;   // argmax: value and first index over the raw logits, kept
        int am_k = -1, am_e = 0; // as (round, element): no per-round index lives across rows
        int am = 0x7fffffff;
        if constexpr (KL > 0) {
            // this wave's LDS rounds have landed once at most the 2 KR memory
            // operations issued after them (KR register-round stores, then the KR
            // register loads) are outstanding; the target element's store, thread
            // 0's row outputs and ignored rows' stores come later still
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * KR) : "memory");
        }
        // thread 0: the drawn row and its label, requested now so both have
        // landed by the combine barrier (the draw was issued before the row's
        // register rounds, so it is complete once they are)
        int64_t nx = n;
        if (tid == 0 && drawn) nx = static_cast<int64_t>(G) + tagged_count(ws_rows(a.workspace), draw, tag);
        int64_t ynx = 0;
        if constexpr (!ARGMAX)
            if (tid == 0 && nx < n) ynx = a.labels[nx];
        // one round of pass A; MK: the round may hold a boundary vector of an
        // unaligned row's window (its first or last round), whose elements of
        // other rows are masked
        auto pa_round = [&](auto mk, int k, const u32x4 &vk) {
            constexpr bool MK = decltype(mk)::value;
            const int idx = k * NT + tid;
            // unaligned rows: the elements of this vector that belong to the
            // row (all but in the first and the last vector of the window)
            unsigned vmask = (1u << E) - 1u;
            if constexpr (MK) {
                int p0 = idx * E - off;   // row position of element 0 (opaque: not hoisted per round)
                asm volatile("" : "+v"(p0));
#pragma unroll
                for (int e = 0; e < E; ++e)
                    if (p0 + e < 0 || p0 + e >= Vi) vmask &= ~(1u << e);
            }
            // z = x, or with the softcap z = T - 2 T r (r = 1 / (1 + e^{2x/T})):
            // then the exponent of z is one fma on r and max z = z(min r)
            // (the fma is monotone in r), so z itself is never formed.
            // Masked elements take x = -inf (r = +inf): no weight, never the max.
            float x[E], z[E];
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const bool in = !MK || ((vmask >> e) & 1u);
                x[e] = in ? EL::get(vk, e) : -INFINITY;
                z[e] = SOFTCAP ? (in ? cap.r_of(x[e]) : INFINITY) : x[e];
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
                if (xmax > amv) {                 // rounds come in index order: keep the first
                    // (rare once the running maximum has settled: the search
                    // for the element runs only then)
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
                if constexpr (MK) {
                    float t = 0.0f;
#pragma unroll
                    for (int e = 0; e < E; ++e)
                        if ((vmask >> e) & 1u) t += SOFTCAP ? fmaf(-2.0f * a.softcap, z[e], a.softcap) : z[e];
                    zs += t;
                } else {
                    float t = z[0];
#pragma unroll
                    for (int e = 1; e < E; ++e) t += z[e];
                    zs += SOFTCAP ? fmaf(-2.0f * a.softcap, t, E * a.softcap) : t;
                }
            }
            const float mn = fmaxf(m, rmax);
            const float mnL = mn * kLog2e;
            float part = 0.0f;
            float ex[E];
            if constexpr (SOFTCAP) {
                const float b = fmaf(a.softcap, kLog2e, -mnL);
#pragma unroll
                for (int e = 0; e < E; ++e) ex[e] = exp2_fast(fmaf(z[e], capk, b));
            } else if constexpr (BF16) {
#pragma unroll
                for (int e = 0; e < E; ++e) ex[e] = exp2_fast(fmaf(z[e], kLog2e, -mnL));
            } else {
                // fp32 rows: every weight relative to the running max itself
                // (z - m is exact where the weight matters), not to an fp32
                // rounding of m log2 e
#pragma unroll
                for (int e = 0; e < E; ++e) ex[e] = exp2_fast((z[e] - mn) * kLog2e);
            }
            if (k == ky) {
                // the target's round (uniform branch, taken once per row); the
                // asm keeps it a branch instead of per-element selects everywhere
                asm volatile("");
                if (owner) {
                    float sel = x[0];
#pragma unroll
                    for (int e = 1; e < E; ++e)
                        if (e == ey) sel = x[e];
                    sh_xy[pb] = sel;
#pragma unroll
                    for (int e = 0; e < E; ++e)
                        if (e == ey) ex[e] = 0.0f;
                }
            }
            part = ex[0];
#pragma unroll
            for (int e = 1; e < E; ++e) part += ex[e];
            s = fmaf(s, exp2_fast(BF16 || SOFTCAP ? fmaf(m, kLog2e, -mnL) : (m - mn) * kLog2e), part);
            m = mn;
        };
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int idx = k * NT + tid;
            // whole rounds need no per-lane test (uniform check first)
            if ((k + 1) * NT <= nv || idx < nv) {
                const u32x4 vk = round_vec(k);
                if constexpr (UA) {
                    if (k == 0 || k == k_last) pa_round(std::true_type{}, k, vk);
                    else pa_round(std::false_type{}, k, vk);
                } else {
                    pa_round(std::false_type{}, k, vk);
                }
            }
        }
        // combine the threads' (m, s) pairs, then the argmax and sum z
        {
            float mw = m, sw = s;
            wave_lse(mw, sw);   // DPP exchanges, no LDS round trips
            if ((tid & 63) == 0) {
                sh_m[pb][tid >> 6] = mw;
                sh_s[pb][tid >> 6] = sw;
            }
            if constexpr (ARGMAX) {
                am = am_k < 0 ? 0x7fffffff : (am_k * NT + tid) * E + am_e - off;
                wave_argmax_dpp(amv, am);
                if ((tid & 63) == 0) {
                    sh_z[pb][tid >> 6] = amv;
                    sh_i[pb][tid >> 6] = am;
                }
            }
            if constexpr (SMOOTH) {
                zs = wave_sum_dpp(zs);
                if ((tid & 63) == 0) sh_zs[pb][tid >> 6] = zs;
            }
            if (tid == 0) {
                // resolve the schedule: without the argmax, ignored rows are
                // not read here; they are zeroed at the end of the call by the
                // workgroups that have run out of rows
                if constexpr (!ARGMAX) {
                    for (int skips = 0; nx < n && !valid_label(ynx) && skips < kSkipMax; ++skips) {
                        nx = static_cast<int64_t>(G) + tagged_draw(ws_rows(a.workspace), tag);
                        if (nx < n) ynx = a.labels[nx];
                    }
                }
                sh_next[pb] = nx;
            }
            __syncthreads();
            float M = sh_m[pb][0];
#pragma unroll
            for (int w = 1; w < NWAVE; ++w) M = fmaxf(M, sh_m[pb][w]);
            float S0 = 0.0f;
#pragma unroll
            for (int w = 0; w < NWAVE; ++w) S0 += sh_s[pb][w] * exp2_fast((sh_m[pb][w] - M) * kLog2e);
            m = M;
            s = S0;
            if constexpr (ARGMAX) {
                amv = sh_z[pb][0];
                am = sh_i[pb][0];
#pragma unroll
                for (int w = 1; w < NWAVE; ++w) argmax_combine(amv, am, sh_z[pb][w], sh_i[pb][w]);
                if (tid == 0 && valid && am == y) ++correct;
            }
            if constexpr (SMOOTH) {
                float t = sh_zs[pb][0];
#pragma unroll
                for (int w = 1; w < NWAVE; ++w) t += sh_zs[pb][w];
                zs = t;
            }
        }
        const float xy = sh_xy[pb];
        const float Mz = m;
        const float zy = SOFTCAP ? cap.z_of_r(cap.r_of(xy)) : xy;
        const float e_y = exp2_fast((zy - Mz) * kLog2e);
        const float S = s + e_y;
        const float lse = Mz + logf(S);
        // thread 0's row outputs are stored only after the next row's loads
        // are out, so that the wait on the register rounds at the start of
        // pass B never includes a store's round trip
        float loss = lse - (1.0f - eps) * zy;
        if constexpr (SMOOTH) loss -= eps * invV * zs;
        if (!valid) loss = 0.0f;

        // ---- pass B: gradient over the logits.  |s_i| is folded into the
        // exponent (exp(z - lse + ln|s_i|)) and its sign applied afterwards
        nxt = sh_next[pb];
        const __amdgpu_buffer_rsrc_t rn = row_rsrc(nxt, nxt < n);
        const float ascale = fabsf(scale);
        const bool negate = scale < 0.0f;
        const float l2s = log2f(ascale);                  // -inf when the scale is 0
        const float epsV = SMOOTH ? eps * invV * ascale : 0.0f;
        const float lseL = lse * kLog2e - l2s;
        // fp32 rows: the exponent is (x - M) log2 e + (log2|s_i| - log2 S), like
        // pass A's weights, so the row max never passes through an fp32 rounding
        // of LSE or of M log2 e (at |x| ~ 4e3 their ulp, 5e-4, would be a relative
        // error in every p_j).  bf16 rows keep the one-fma form: that rounding is
        // far below half a bf16 ulp.
        const float l2rel = l2s - log2f(S);
        const float capb2 = (a.softcap - lse) * kLog2e + l2s;
        float gy = scale * (eps - s / S - (SMOOTH ? eps * invV : 0.0f));   // s_i (p_y - (1 - eps) - eps/V)
        if constexpr (SOFTCAP) {
            float ry, qy;
            cap.r_q(xy, ry, qy);
            gy *= Cap::chain(ry, qy);
        }
        // an ignored row's gradient is +0 everywhere (0 times a negative factor
        // would store -0 here, while the end-of-call zeroing stores +0)
        if (!valid) gy = 0.0f;
        opaque_regs(v);
        // one round of pass B; MK as in pass A: a boundary vector's lane stores
        // the row's own elements of it one at a time
        auto grad_round_mk = [&](auto mk, int k) {
            constexpr bool MK = decltype(mk)::value;
            const u32x4 vk = round_vec(k);
            float g[E];
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const float x = EL::get(vk, e);
                if constexpr (SOFTCAP) {
                    // chain 4 r (1 - r): the 4 rides in the exponent (capb2 + 2)
                    float r, q;
                    cap.r_q(x, r, q);
                    const float p4 = exp2_fast(fmaf(r, capk, capb2 + 2.0f));   // 4 |s_i| p_j
                    g[e] = (SMOOTH ? p4 - 4.0f * epsV : p4) * (r * q);
                } else {
                    const float p = BF16 ? exp2_fast(fmaf(x, kLog2e, -lseL))          // |s_i| p_j
                                         : exp2_fast(fmaf(x - Mz, kLog2e, l2rel));
                    g[e] = SMOOTH ? p - epsV : p;
                }
            }
            if (negate) {
                asm volatile("");
#pragma unroll
                for (int e = 0; e < E; ++e) g[e] = -g[e];
            }
            if constexpr (MK) {
                const bool bnd = boundary(k * NT + tid, off, nv);
                const u32x4 pk = EL::pack(g);
                store_round(k, rp, pk, bnd);
                if (bnd) store_elems(rp, k * NT + tid, off, pk);
            } else {
                store_round(k, rp, EL::pack(g));
            }
            // keep the rounds in order: hoisted loads or conversions of later
            // rounds would hold extra row data in registers
            __builtin_amdgcn_sched_barrier(0);
        };
        auto grad_round = [&](int k) { grad_round_mk(std::integral_constant<bool, UA>{}, k); };
        // the LDS rounds, then the next row's LDS rounds go out (this wave read
        // its slots before computing the stores above, and no other wave uses them).
        // Without the softcap the workgroup first lets its LDS-round stores
        // drain and meets at a barrier, so the next row's loads leave together
        // (1.3% faster on the label-smoothing workload).  The softcap variants
        // are VALU-bound: they lose 5% to that barrier, and there each round's
        // load for the next row goes out right after the round's gradient store,
        // so the next row arrives while this one is still being computed (2.5%
        // faster at 4096 x 202048; on the memory-bound rows the grouped order is
        // 1-5% faster).  Either order leaves 2 KR memory operations behind the
        // last LDS-round load, which the wait at the top of pass A counts on.
#pragma unroll
        for (int k = 0; k < KL; ++k) {
            grad_round(k);
            if constexpr (SOFTCAP) issue_round(k, rn);
        }
        if constexpr (KL > 0 && !SOFTCAP) __syncthreads();
        if constexpr (!SOFTCAP) {
#pragma unroll
            for (int k = 0; k < KL; ++k) {
                issue_round(k, rn);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // the row after the next (none to draw once the schedule has run out: a
        // draw still in flight would delay this workgroup's final publish)
        if (tid == 0) {
            drawn = nxt < n;
            if (drawn) draw = tagged_inc(ws_rows(a.workspace));
        }
        __builtin_amdgcn_sched_barrier(0);
        // the register rounds, then the next row's register rounds
#pragma unroll
        for (int k = KL; k < K; ++k) {
            grad_round(k);
            if constexpr (SOFTCAP) {   // as for the LDS rounds
                issue_round(k, rn);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        if constexpr (!SOFTCAP) {
#pragma unroll
            for (int k = KL; k < K; ++k) {
                issue_round(k, rn);   // in the order pass A consumes them
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // the target element's own gradient replaces what its round stored
        // (one thread, after that round's store, to the same address)
        if (owner) EL::template store_one<kNonTemporal>(rp, y + off, gy);
        if (tid == 0) {
            store_through(a.loss_tok + row, loss);
            if constexpr (ARGMAX) a.argmax_out[row] = am;
        }
    }

    // ---- without the argmax, the ignored rows the walk stepped over (all at or
    // past row G: the first rows are carried through) are zeroed last, in
    // chunks of kZeroChunk rows drawn from their own counter, by the
    // workgroups that have run out of rows: this moves the stores into the
    // time that workgroups finishing early would otherwise sit idle.  An
    // ignored row that was also carried through the row loop (past kSkipMax
    // skips) gets zeros twice: the same bytes.
    if constexpr (!ARGMAX) {
        if (tid == 0 && G < n) tagged_claim(ws_zero_chunks(a.workspace), tag);
        for (int q = 0; G < n; q ^= 1) {
            if (tid == 0) sh_chunk[q] = tagged_draw(ws_zero_chunks(a.workspace), tag);
            __syncthreads();
            const int64_t c0 = static_cast<int64_t>(G) + static_cast<int64_t>(sh_chunk[q]) * kZeroChunk;
            if (c0 >= n) break;
            if (tid < 64) {
                const int64_t r = c0 + tid;
                const bool ign = r < n && !valid_label(a.labels[r]);
                const unsigned long long m = __ballot(ign);
                if (tid == 0) sh_ign[q] = m;
            }
            __syncthreads();
            for (unsigned long long m = sh_ign[q]; m; m &= m - 1) zero_row(c0 + __builtin_ctzll(m));
        }
    }

    // ---- publish this workgroup's n_correct; the last workgroup folds the
    // per-token losses and these counts.  Both were written through to memory
    // (system-scope stores) and are acknowledged before the ticket is taken,
    // and the last workgroup reads them past its own L2.
    if (tid == 0) {
        __hip_atomic_store(ws_correct(a.workspace) + blockIdx.x, correct, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_SYSTEM);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        tagged_claim(ws_ticket(a.workspace), tag);
        const unsigned t = tagged_draw(ws_ticket(a.workspace), tag);
        sh_flag = t == static_cast<unsigned>(G) - 1u;
    }
    __syncthreads();
    if (!sh_flag) return;
    long long n_valid, n_bad;
    count_labels_read(sh_c, n_valid, n_bad);
    // fixed order: thread t sums rows t, t + NT, ... in fp64, then the waves'
    // sums are combined in wave order.  Eight loads go out before the first
    // is added, so the fold waits for one round trip per eight rows per thread.
    double acc = 0.0;
    // this thread's first n_correct partial goes out with the first batch of losses
    // (clamped like them, masked when added)
    long long cor = __hip_atomic_load(ws_correct(a.workspace) + (tid < G ? tid : 0), __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_SYSTEM);
    constexpr int kFold = 8;
    for (int64_t r0 = 0; r0 < n; r0 += kFold * NT) {
        float lv[kFold];
        // (unconditional loads of a clamped row, masked when added: a load
        // under a branch would be waited for at the branch's end)
#pragma unroll
        for (int u = 0; u < kFold; ++u) {
            const int64_t r = r0 + u * NT + tid;
            lv[u] = __uint_as_float(__hip_atomic_load(reinterpret_cast<unsigned *>(a.loss_tok) + (r < n ? r : n - 1),
                                                      __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM));
        }
#pragma unroll
        for (int u = 0; u < kFold; ++u)
            if (r0 + u * NT + tid < n) acc += static_cast<double>(lv[u]);
    }
    if (tid >= G) cor = 0;
    for (int w = tid + NT; w < G; w += NT)
        cor += __hip_atomic_load(ws_correct(a.workspace) + w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    acc = wave_sum_d(acc);
    cor = wave_sum_ll(cor);
    if ((tid & 63) == 0) {
        sh_d[tid >> 6] = acc;
        sh_k[tid >> 6] = cor;
    }
    __syncthreads();
    if (tid == 0) {
        double tot = 0.0;
        long long c = 0;
        for (int w = 0; w < NWAVE; ++w) {
            tot += sh_d[w];
            c += sh_k[w];
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
        *ws_ticket(a.workspace) = 0ull;
        *ws_rows(a.workspace) = 0ull;
        *ws_zero_chunks(a.workspace) = 0ull;
    }
}

// Host-side launch of one (dtype, KR, KL) family: picks the feature variant and
// sizes the persistent grid to the workgroups the CUs hold at once.
template <bool BF16, int KR, int KL, bool S, bool A, bool M, bool UA>
hipError_t launch_variant(const CEArgs &a, int max_groups, hipStream_t st) {
    static int per_cu = 0;   // resident workgroups per CU (same for every gfx950 device)
    if (per_cu == 0) {
        int nb = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, ce_rows_kernel<BF16, KR, KL, S, A, M, UA>, NT, 0) !=
                hipSuccess || nb < 1)
            nb = 1;
        per_cu = nb;
    }
    int64_t grid = static_cast<int64_t>(max_groups) * per_cu;
    if (grid > a.n) grid = a.n;
    if (grid > kMaxRowGroups) grid = kMaxRowGroups;
    hipLaunchKernelGGL((ce_rows_kernel<BF16, KR, KL, S, A, M, UA>), dim3(static_cast<unsigned>(grid)), dim3(NT), 0,
                       st, a);
    return hipGetLastError();
}

template <bool BF16, int KR, int KL, bool UA>
hipError_t launch_rows(const CEArgs &a, int max_groups, hipStream_t st) {
    const bool sc = a.softcap > 0.0f, am = a.argmax_out != nullptr, sm = a.eps != 0.0f;
#define LCE_ROWS(S, A, M) return launch_variant<BF16, KR, KL, S, A, M, UA>(a, max_groups, st)
    if (sc) {
        if (am) { if (sm) LCE_ROWS(true, true, true); else LCE_ROWS(true, true, false); }
        else    { if (sm) LCE_ROWS(true, false, true); else LCE_ROWS(true, false, false); }
    } else {
        if (am) { if (sm) LCE_ROWS(false, true, true); else LCE_ROWS(false, true, false); }
        else    { if (sm) LCE_ROWS(false, false, true); else LCE_ROWS(false, false, false); }
    }
#undef LCE_ROWS
}

}  // namespace dev
}  // namespace lce
