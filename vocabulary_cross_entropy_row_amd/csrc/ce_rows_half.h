// Half-row cross-entropy kernel (gfx950): two workgroups per row.
//
// The per-row arithmetic is that of ce_rows.h (the same loss, gradient,
// softcap, label smoothing and argmax, after Liger-Kernel PR "Add Megatron-LM
// cross-entropy integration", Summary; Megatron-LM PR "Add opt-in Liger
// vocab-parallel cross entropy", "What does this PR do?"; Liger-Kernel PR "Add
// Liger Kernel support for Muse Glimmer", Details/Softcap).  What differs is
// the unit of work.  Workgroups 2j and 2j+1 form pair j and take the same rows:
// the first (the leader) half 0 of each row, i.e. its first ceil(V / E / 2)
// 16-byte vectors, the second (the follower) half 1.  Each workgroup reduces
// its half, and the two exchange their halves' statistics (running max, sum of
// exponentials without the target, target logit, sum z, argmax) through one
// record each in the workspace; both then combine the two records in the same
// order, so both halves' gradients use bit-identical row statistics.
//
// A workgroup holds two half rows at once, one in LDS and one in VGPRs, so the
// loads of the next half row stream in while the current one is reduced and
// its gradient stored: half-row units halve the fixed cost at both ends of a
// call (the first unit lands sooner, the last ones finish closer together).
//
// Fifteen waves hold the data (rounds of 960 vectors).  The sixteenth, the
// control wave, draws rows (the leader's), publishes this workgroup's record,
// polls the partner's and writes the row outputs.  On gfx950 loads and stores
// share one in-order vmcnt per wave, so a poll issued by a data wave would
// wait for that wave's in-flight row loads; the control wave has none.
//
// Records: per workgroup two slots (by iteration parity), eight 64-bit words
// each, every word a 32-bit payload under a 32-bit key (launch, iteration).  A
// reader takes a record only when every word it needs carries the key, so no
// ordering between the words is needed; it then clears the record's first
// word, and waits for that clear before it publishes its next record, which
// the partner must read before it can reuse the slot.  A finished call
// therefore leaves no readable record.
//
// Progress: both workgroups of a pair publish before they wait, and rows are
// drawn by the leader and passed to the follower in the leader's record, so
// the two take the same rows in the same order and a pair can only wait for a
// partner that is not yet running.  The poll is bounded nonetheless: past
// kHalfPollMax polls the row's statistics become NaN, so a partner that never
// arrives shows in the outputs instead of stalling the device.
#pragma once

#include <type_traits>

#include "ce_device.h"

namespace lce {
namespace dev {

constexpr int kHalfDataWaves = 15;
constexpr int kHalfData = kHalfDataWaves * 64;   // data threads (one 16-byte vector each per round)
constexpr unsigned kHalfPollMax = 1u << 20;   // about a second of polls
constexpr int kHalfZeroChunk = 64;

// Record words: 0 max, 1 sum of exponentials, 2 target logit, 3 next row
// (leader), 4 sum z, 5 argmax value, 6 argmax index.
__device__ __forceinline__ unsigned half_key(unsigned tag, unsigned it) {
    return 0x80000000u | ((tag & 0x7fffffu) << 8) | (it & 0xffu);
}
__device__ __forceinline__ void rec_put(unsigned long long *w, unsigned key, unsigned payload) {
    __hip_atomic_store(w, (static_cast<unsigned long long>(key) << 32) | payload, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ unsigned long long rec_get(const unsigned long long *w) {
    return __hip_atomic_load(const_cast<unsigned long long *>(w), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// Three 16-byte LDS reads that wait for themselves.  The row slot in LDS is
// filled by direct-to-LDS loads; a compiler-visible LDS read would also wait
// for those still in flight (it cannot tell the slots apart), so the slot is
// read here, after an explicit wait for exactly its own loads.
__device__ __forceinline__ void lds_read3(u32x4 &x0, u32x4 &x1, u32x4 &x2, unsigned p0, unsigned p1, unsigned p2) {
    asm volatile("ds_read_b128 %0, %3\n\tds_read_b128 %1, %4\n\tds_read_b128 %2, %5\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(x0), "=&v"(x1), "=&v"(x2)
                 : "v"(p0), "v"(p1), "v"(p2)
                 : "memory");
}
// A workgroup barrier for LDS traffic only: this wave's LDS operations are
// complete, then all waves meet.  (__syncthreads() also orders the direct-to-LDS
// row loads in flight, i.e. waits for them.)
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}
// Wait until at most N vector-memory operations of this wave are in flight,
// tied to a register round so that its uses stay behind the wait.
template <int N>
__device__ __forceinline__ void wait_round(u32x4 &x) {
    asm volatile("s_waitcnt vmcnt(%1)" : "+v"(x) : "n"(N));
}

template <bool BF16, int KH, bool SOFTCAP, bool ARGMAX, bool SMOOTH>
__global__ __launch_bounds__(NT) void ce_half_kernel(CEArgs a) {
    using EL = Elt<BF16>;
    constexpr int E = EL::E;
    constexpr int ND = kHalfData;
    constexpr int NDW = kHalfDataWaves;
    __shared__ u32x4 lds_rows[KH * ND];
    __shared__ float sh_m[NDW], sh_s[NDW], sh_z[NDW], sh_zs[NDW];
    __shared__ int sh_i[NDW];
    __shared__ long long sh_c[2][NDW];     // label count partials (valid, bad) of the data waves
    __shared__ long long sh_nbad;
    __shared__ long long sh_k[NWAVE];
    __shared__ double sh_d[NWAVE];
    __shared__ float sh_xy;
    // what the control wave hands the data waves at each exchange: row max, sum
    // of exponentials without the target, sum z, target logit, next row (int64),
    // valid-label count (int64)
    __shared__ __align__(16) unsigned sh_bc[8];
    __shared__ unsigned long long sh_ign;
    __shared__ unsigned sh_chunk;
    __shared__ int sh_flag;

    const int tid = threadIdx.x;
    // the control wave (a wave-uniform test: each wave runs one of the two loops
    // below, with the same barriers in the same order)
    const bool ctl = __builtin_amdgcn_readfirstlane(tid >= ND ? 1 : 0) != 0;
    const bool ctl0 = tid == ND;
    const int wave_base = tid & ~63;
    const int nvec = static_cast<int>(a.V / E);
    const int hv0 = (nvec + 1) >> 1;
    const int G = gridDim.x;   // even
    const int P = G >> 1;
    const int pair = static_cast<int>(blockIdx.x >> 1);
    const int h = static_cast<int>(blockIdx.x & 1);
    const int hv = h ? nvec - hv0 : hv0;   // vectors of this workgroup's half
    const int hoff = h ? hv0 : 0;          // its first vector
    const int64_t n = a.n;
    const float eps = a.eps;
    const float invV = 1.0f / static_cast<float>(a.V);
    const Cap cap{SOFTCAP ? 2.0f * kLog2e / a.softcap : 0.0f, a.softcap};
    const float capk = -2.0f * a.softcap * kLog2e;
    const u32x4 zero4 = {0u, 0u, 0u, 0u};
    typedef const __attribute__((address_space(4))) int64_t *clabels_t;
    typedef const __attribute__((address_space(4))) float *cfloat_t;
    const clabels_t lab = (clabels_t)a.labels;
    const cfloat_t gout = (cfloat_t)a.grad_out;
    unsigned long long *const recs =
        reinterpret_cast<unsigned long long *>(static_cast<char *>(a.workspace) + ce_records_offset(n));

    auto valid_label = [&](int64_t y) { return y != a.ignore_index && y >= 0 && y < a.V; };

    // this workgroup's half of row r (an empty descriptor when there is none:
    // loads through it return zeros and stores are dropped, without touching memory)
    auto half_rsrc = [&](int64_t r, bool live) {
        return __builtin_amdgcn_make_buffer_rsrc(
            static_cast<char *>(a.logits) + (live ? r * a.ld * EL::bytes + static_cast<int64_t>(hoff) * 16 : 0), 0,
            live ? static_cast<uint32_t>(hv) * 16u : 0u, kBufferWord3);
    };
    const int voff = tid * 16;

    // slot 0: KH rounds in LDS; slot 1: KH rounds in VGPRs
    u32x4 v[KH];
    auto issue_lds = [&](int k, __amdgpu_buffer_rsrc_t src) {
        typedef __attribute__((address_space(3))) void *lptr;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (lptr)(&lds_rows[k * ND + wave_base]), 16, voff, k * ND * 16, 0,
                                                 kNonTemporal);
    };
    auto issue_reg = [&](int k, __amdgpu_buffer_rsrc_t src) {
        v[k] = __builtin_amdgcn_raw_buffer_load_b128(src, voff, k * ND * 16, kNonTemporal);
    };
    // the round offset rides in the VGPR offset (see ce_rows.h: with it in
    // soffset, gfx950 lets the next VALU write overtake the store's data read)
    auto store_round = [&](int k, __amdgpu_buffer_rsrc_t dst, u32x4 val) {
        int vo = voff;
        asm volatile("" : "+v"(vo));
        __builtin_amdgcn_raw_buffer_store_b128(val, dst, vo + k * ND * 16, 0, kNonTemporal);
    };

    // Row and label data of a half row (shared by both loops).
    struct RowInfo {
        bool valid;
        int y, ey, hy, vh, ky, ty;
    };
    auto row_info = [&](int64_t r) {
        RowInfo q;
        const int64_t y64 = lab[r];
        q.valid = valid_label(y64);
        q.y = q.valid ? static_cast<int>(y64) : 0;
        // the target: vector vy in half hy; its vector vh within the half, round ky
        // (-1 when it lies in the other half) and thread ty
        const int vy = q.y / E;
        q.ey = q.y % E;
        q.hy = vy >= hv0 ? 1 : 0;
        q.vh = vy - (q.hy ? hv0 : 0);
        q.ky = q.hy == h ? q.vh / ND : -1;
        q.ty = q.vh % ND;
        return q;
    };
    auto uniform64 = [](int64_t x) {
        const uint64_t u = static_cast<uint64_t>(x);
        const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u));
        const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u >> 32));
        return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
    };

    // static rows: pair j takes rows j and P + j; then the leader draws rows
    // from G on and hands each to the follower in its record
    const unsigned tag = launch_tag();
    const int64_t row0 = pair;
    const int64_t row1 = P + pair < n ? P + pair : n;
    long long correct = 0;

    if (ctl) {
        // ================= control wave =================
        const int lane = tid - ND;
        // labels from 2 * ND on (the data waves count the first 2 * ND), sixteen
        // loads in flight per lane
        long long cv = 0, cb = 0;
        for (int64_t i0 = 2 * ND; i0 < a.count_n; i0 += 16 * 64) {
            int64_t yl[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const int64_t i = i0 + u * 64 + lane;
                yl[u] = i < a.count_n ? a.count_labels[i] : a.ignore_index;
            }
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                if (yl[u] != a.ignore_index) {
                    if (yl[u] >= 0 && yl[u] < a.V) ++cv;
                    else ++cb;
                }
            }
        }
        cv = wave_sum_ll(cv);
        cb = wave_sum_ll(cb);
        // the leader's first drawn row, resolved ahead of need
        bool drawing = G < n;
        int64_t drawn_row = n;
        auto draw = [&]() {
            drawn_row = n;
            while (drawing) {
                const int64_t r = static_cast<int64_t>(G) + tagged_draw(ws_rows(a.workspace), tag);
                if (r >= n) {
                    drawing = false;
                    break;
                }
                // without the argmax, ignored rows are skipped (zeroed at the end)
                if (ARGMAX || valid_label(a.labels[r])) {
                    drawn_row = r;
                    break;
                }
            }
        };
        if (ctl0 && h == 0 && drawing) {
            tagged_claim(ws_rows(a.workspace), tag);
            draw();
        }
        unsigned it = 0;
        for (int64_t r = row0, r1 = row1; r < n; ++it) {
            const RowInfo q = row_info(r);
            lds_barrier();   // this half's partials are in LDS
            if (it == 0) {
                // the label counts: the data waves' partials and this wave's
                long long tv = cv, tb = cb;
#pragma unroll
                for (int w = 0; w < NDW; ++w) {
                    tv += sh_c[0][w];
                    tb += sh_c[1][w];
                }
                if (ctl0) {
                    sh_bc[6] = static_cast<unsigned>(static_cast<unsigned long long>(tv));
                    sh_bc[7] = static_cast<unsigned>(static_cast<unsigned long long>(tv) >> 32);
                    sh_nbad = tb;
                }
            }
            float mh = sh_m[0];
#pragma unroll
            for (int w = 1; w < NDW; ++w) mh = fmaxf(mh, sh_m[w]);
            float sH = 0.0f;
#pragma unroll
            for (int w = 0; w < NDW; ++w) sH += sh_s[w] * exp2_fast((sh_m[w] - mh) * kLog2e);
            float zh = 0.0f, amvh = -INFINITY;
            int amh = 0x7fffffff;
            if constexpr (SMOOTH) {
#pragma unroll
                for (int w = 0; w < NDW; ++w) zh += sh_zs[w];
            }
            if constexpr (ARGMAX) {
                amvh = sh_z[0];
                amh = sh_i[0];
#pragma unroll
                for (int w = 1; w < NDW; ++w) argmax_combine(amvh, amh, sh_z[w], sh_i[w]);
            }
            const float xyh = q.hy == h ? sh_xy : 0.0f;
            if (ctl0) {
                const unsigned key = half_key(tag, it);
                unsigned long long *mine = recs + (static_cast<size_t>(blockIdx.x) * 2 + (it & 1u)) * 8;
                unsigned long long *theirs = recs + (static_cast<size_t>(blockIdx.x ^ 1u) * 2 + (it & 1u)) * 8;
                // the clear of the partner's previous record has landed
                wait_vmem_all();
                rec_put(mine + 0, key, __float_as_uint(mh));
                rec_put(mine + 1, key, __float_as_uint(sH));
                rec_put(mine + 2, key, __float_as_uint(xyh));
                if (h == 0) rec_put(mine + 3, key, static_cast<unsigned>(drawn_row));
                if constexpr (SMOOTH) rec_put(mine + 4, key, __float_as_uint(zh));
                if constexpr (ARGMAX) {
                    rec_put(mine + 5, key, __float_as_uint(amvh));
                    rec_put(mine + 6, key, static_cast<unsigned>(amh));
                }
                unsigned long long w[7] = {0, 0, 0, 0, 0, 0, 0};
                bool ok = false;
                for (unsigned poll = 0; poll < kHalfPollMax; ++poll) {
                    w[0] = rec_get(theirs + 0);
                    w[1] = rec_get(theirs + 1);
                    w[2] = rec_get(theirs + 2);
                    if (h == 1) w[3] = rec_get(theirs + 3);
                    if constexpr (SMOOTH) w[4] = rec_get(theirs + 4);
                    if constexpr (ARGMAX) {
                        w[5] = rec_get(theirs + 5);
                        w[6] = rec_get(theirs + 6);
                    }
                    bool all = true;
#pragma unroll
                    for (int u = 0; u < 7; ++u) {
                        const bool used = u < 3 || (u == 3 && h == 1) || (u == 4 && SMOOTH) || (u >= 5 && ARGMAX);
                        if (used && static_cast<unsigned>(w[u] >> 32) != key) all = false;
                    }
                    if (all) {
                        ok = true;
                        break;
                    }
                    __builtin_amdgcn_s_sleep(2);
                }
                // the record is consumed: clear its first word
                __hip_atomic_store(theirs, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
                const float pm = __uint_as_float(static_cast<unsigned>(w[0]));
                const float ps = __uint_as_float(static_cast<unsigned>(w[1]));
                const float pxy = __uint_as_float(static_cast<unsigned>(w[2]));
                const float pz = __uint_as_float(static_cast<unsigned>(w[4]));
                const float pamv = __uint_as_float(static_cast<unsigned>(w[5]));
                const int pam = static_cast<int>(static_cast<unsigned>(w[6]));
                // combine in half order on both sides
                const float m0 = h ? pm : mh, s0 = h ? ps : sH, m1 = h ? mh : pm, s1 = h ? sH : ps;
                float M = fmaxf(m0, m1);
                const float S = s0 * exp2_fast((m0 - M) * kLog2e) + s1 * exp2_fast((m1 - M) * kLog2e);
                if (!ok) M = __builtin_nanf("");
                const float zsum = h ? pz + zh : zh + pz;
                const float xy = q.hy == h ? xyh : pxy;
                const int64_t nx = h ? static_cast<int64_t>(static_cast<unsigned>(w[3])) : drawn_row;
                const int64_t nxc = nx < n ? nx : n;
                sh_bc[0] = __float_as_uint(M);
                sh_bc[1] = __float_as_uint(S);
                sh_bc[2] = __float_as_uint(zsum);
                sh_bc[3] = __float_as_uint(xy);
                sh_bc[4] = static_cast<unsigned>(static_cast<uint64_t>(nxc));
                sh_bc[5] = static_cast<unsigned>(static_cast<uint64_t>(nxc) >> 32);
                if (h == 0) {
                    // the row outputs
                    float amv = amvh;
                    int am = amh;
                    if constexpr (ARGMAX) argmax_combine(amv, am, pamv, pam);
                    const float zy = SOFTCAP ? cap.z_of_r(cap.r_of(xy)) : xy;
                    const float e_y = exp2_fast((zy - M) * kLog2e);
                    const float lse = M + logf(S + e_y);
                    float loss = lse - (1.0f - eps) * zy;
                    if constexpr (SMOOTH) loss -= eps * invV * zsum;
                    if (!q.valid) loss = 0.0f;
                    store_through(a.loss_tok + r, loss);
                    if constexpr (ARGMAX) {
                        a.argmax_out[r] = am;
                        if (q.valid && am == q.y) ++correct;
                    }
                }
            }
            lds_barrier();   // the row statistics and the next row are in LDS
            const int64_t nx = uniform64(static_cast<int64_t>((static_cast<uint64_t>(sh_bc[5]) << 32) | sh_bc[4]));
            if (ctl0 && h == 0) draw();   // the row after that one (idle until the next exchange)
            r = r1;
            r1 = nx;
        }
    } else {
        // ================= data waves =================
        // the first 2 * ND labels are requested ahead of the row loads, so
        // counting them does not wait behind those
        const int64_t yc0 = tid < a.count_n ? a.count_labels[tid] : a.ignore_index;
        const int64_t yc1 = tid + ND < a.count_n ? a.count_labels[tid + ND] : a.ignore_index;
        __builtin_amdgcn_sched_barrier(0);
        {
            const __amdgpu_buffer_rsrc_t s0 = half_rsrc(row0, true);
#pragma unroll
            for (int k = 0; k < KH; ++k) {
                issue_lds(k, s0);
                __builtin_amdgcn_sched_barrier(0);
            }
            const __amdgpu_buffer_rsrc_t s1 = half_rsrc(row1, row1 < n);
#pragma unroll
            for (int k = 0; k < KH; ++k) {
                issue_reg(k, s1);
                __builtin_amdgcn_sched_barrier(0);
            }
            // KH dropped stores: the first LDS half row then has the same 2 KH
            // memory operations behind it as every later one, so one wait count
            // serves all
            const __amdgpu_buffer_rsrc_t none = half_rsrc(0, false);
#pragma unroll
            for (int k = 0; k < KH; ++k) store_round(k, none, zero4);
        }
        {
            long long cv = 0, cb = 0;
            auto count = [&](int64_t y) {
                if (y != a.ignore_index) {
                    if (y >= 0 && y < a.V) ++cv;
                    else ++cb;
                }
            };
            count(yc0);
            count(yc1);
            cv = wave_sum_ll(cv);
            cb = wave_sum_ll(cb);
            if ((tid & 63) == 0) {
                sh_c[0][tid >> 6] = cv;
                sh_c[1][tid >> 6] = cb;
            }
        }
        const float g_all = (a.reduction != 0 && gout) ? gout[0] : 1.0f;

        // One half row: pass A, the exchange (control wave), pass B, then the
        // loads of the half row two steps ahead into the slot just freed.
        auto step = [&](auto in_lds, int64_t r) -> int64_t {
            constexpr bool L = decltype(in_lds)::value;
            const RowInfo q = row_info(r);
            const bool owner = q.ky >= 0 && tid == q.ty;
            const __amdgpu_buffer_rsrc_t rp = half_rsrc(r, true);
            // this thread's LDS address of round k of the LDS slot
            const unsigned lds_base = static_cast<unsigned>(
                reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) u32x4 *)lds_rows)) + tid * 16u;
            auto lds_addr = [&](int k) { return lds_base + static_cast<unsigned>((k < KH ? k : 0) * ND * 16); };
            // register round k has landed once at most 3 KH - 1 - k vector-memory
            // operations are in flight: the rest of its slot's loads, then the LDS
            // slot's stores and loads
            auto wait_reg = [&](int k) {
                if (k == 0) wait_round<3 * KH - 1>(v[0]);
                else if (k == 1) wait_round<3 * KH - 2>(v[1]);
                else if (k == 2) wait_round<3 * KH - 3>(v[2]);
                else if (k == 3) wait_round<3 * KH - 4>(v[3]);
                else if (k == 4) wait_round<3 * KH - 5>(v[4]);
                else if (k == 5) wait_round<3 * KH - 6>(v[5]);
                else if (k == 6) wait_round<3 * KH - 7>(v[6]);
                else if (k == 7) wait_round<3 * KH - 8>(v[7]);
                else if (k == 8) wait_round<3 * KH - 9>(v[8 < KH ? 8 : 0]);
                else if (k == 9) wait_round<3 * KH - 10>(v[9 < KH ? 9 : 0]);
            };
            static_assert(KH <= 10, "wait_reg covers ten register rounds");
            // the slot's rounds (the LDS slot's in groups of three): f(k, round)
            // for each, after its wait when `first`
            auto for_rounds = [&](auto first, auto f) {
                if constexpr (L) {
#pragma unroll
                    for (int g = 0; g < KH; g += 3) {
                        u32x4 t0, t1, t2;
                        lds_read3(t0, t1, t2, lds_addr(g), lds_addr(g + 1), lds_addr(g + 2));
                        f(g, t0);
                        if (g + 1 < KH) f(g + 1, t1);
                        if (g + 2 < KH) f(g + 2, t2);
                    }
                } else {
#pragma unroll
                    for (int k = 0; k < KH; ++k) {
                        if constexpr (decltype(first)::value) wait_reg(k);
                        f(k, v[k]);
                    }
                }
            };
            // ---- pass A over this half.  The LDS slot's loads have landed once at
            // most the 2 KH memory operations issued after them (the register
            // slot's stores and loads) are in flight.
            float m = -FLT_MAX, s = 0.0f, zs = 0.0f, amv = -INFINITY;
            int am_k = -1, am_e = 0;
            if constexpr (L) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * KH) : "memory");
            for_rounds(std::integral_constant<bool, true>{}, [&](int k, const u32x4 &vk) {
                const int idx = k * ND + tid;
                if ((k + 1) * ND <= hv || idx < hv) {
                    float x[E], z[E];
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        x[e] = EL::get(vk, e);
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
                    if (k == q.ky) {
                        asm volatile("");
                        if (owner) {
                            float sel = x[0];
#pragma unroll
                            for (int e = 1; e < E; ++e)
                                if (e == q.ey) sel = x[e];
                            sh_xy = sel;
#pragma unroll
                            for (int e = 0; e < E; ++e)
                                if (e == q.ey) ex[e] = 0.0f;
                        }
                    }
                    float part = ex[0];
#pragma unroll
                    for (int e = 1; e < E; ++e) part += ex[e];
                    s = fmaf(s, exp2_fast(BF16 || SOFTCAP ? fmaf(m, kLog2e, -mnL) : (m - mn) * kLog2e), part);
                    m = mn;
                }
            });
            float mw = m, sw = s;
            wave_lse(mw, sw);
            if ((tid & 63) == 0) {
                sh_m[tid >> 6] = mw;
                sh_s[tid >> 6] = sw;
            }
            if constexpr (ARGMAX) {
                int am = am_k < 0 ? 0x7fffffff : (hoff + am_k * ND + tid) * E + am_e;
                wave_argmax_dpp(amv, am);
                if ((tid & 63) == 0) {
                    sh_z[tid >> 6] = amv;
                    sh_i[tid >> 6] = am;
                }
            }
            if constexpr (SMOOTH) {
                zs = wave_sum_dpp(zs);
                if ((tid & 63) == 0) sh_zs[tid >> 6] = zs;
            }
            lds_barrier();   // partials out; the control wave exchanges
            lds_barrier();   // the row statistics and the next row are in
            // (read with a wait on LDS alone: the compiler would also wait for the
            // direct-to-LDS row loads in flight, which write elsewhere)
            u32x4 b0, b1;
            {
                const unsigned addr = static_cast<unsigned>(
                    reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) unsigned *)sh_bc));
                asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %2 offset:16\n\ts_waitcnt lgkmcnt(0)"
                             : "=v"(b0), "=v"(b1)
                             : "v"(addr)
                             : "memory");
            }
            const int64_t nx = uniform64(static_cast<int64_t>((static_cast<uint64_t>(b1.y) << 32) | b1.x));
            const long long nvalid = static_cast<long long>((static_cast<uint64_t>(b1.w) << 32) | b1.z);

            // ---- pass B over this half
            float red_scale = g_all;
            if (a.reduction == 1) red_scale = nvalid > 0 ? g_all / static_cast<float>(nvalid) : 0.0f;
            const float scale = !q.valid ? 0.0f : (a.reduction == 0 ? (gout ? gout[r] : 1.0f) : red_scale);
            const float Mz = __uint_as_float(b0.x);
            const float sx = __uint_as_float(b0.y);
            const float xy = __uint_as_float(b0.w);
            const float zy = SOFTCAP ? cap.z_of_r(cap.r_of(xy)) : xy;
            const float e_y = exp2_fast((zy - Mz) * kLog2e);
            const float S = sx + e_y;
            const float lse = Mz + logf(S);
            const float ascale = fabsf(scale);
            const bool negate = scale < 0.0f;
            const float l2s = log2f(ascale);
            const float epsV = SMOOTH ? eps * invV * ascale : 0.0f;
            const float lseL = lse * kLog2e - l2s;
            const float l2rel = l2s - log2f(S);
            const float capb2 = (a.softcap - lse) * kLog2e + l2s;
            float gy = scale * (eps - sx / S - (SMOOTH ? eps * invV : 0.0f));
            if constexpr (SOFTCAP) {
                float ry, qy;
                cap.r_q(xy, ry, qy);
                gy *= Cap::chain(ry, qy);
            }
            if (!q.valid) gy = 0.0f;
            if constexpr (!L) opaque_regs(v);
            for_rounds(std::integral_constant<bool, false>{}, [&](int k, const u32x4 &vk) {
                float g[E];
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const float x = EL::get(vk, e);
                    if constexpr (SOFTCAP) {
                        float rr, qq;
                        cap.r_q(x, rr, qq);
                        const float p4 = exp2_fast(fmaf(rr, capk, capb2 + 2.0f));
                        g[e] = (SMOOTH ? p4 - 4.0f * epsV : p4) * (rr * qq);
                    } else {
                        const float p = BF16 ? exp2_fast(fmaf(x, kLog2e, -lseL))
                                             : exp2_fast(fmaf(x - Mz, kLog2e, l2rel));
                        g[e] = SMOOTH ? p - epsV : p;
                    }
                }
                if (negate) {
                    asm volatile("");
#pragma unroll
                    for (int e = 0; e < E; ++e) g[e] = -g[e];
                }
                store_round(k, rp, EL::pack(g));
                __builtin_amdgcn_sched_barrier(0);
            });
            // the target element's own gradient replaces what its round stored
            if (owner) EL::template store_one<kNonTemporal>(rp, q.vh * E + q.ey, gy);
            // the half row two steps ahead, into the slot just freed
            const __amdgpu_buffer_rsrc_t rn = half_rsrc(nx, nx < n);
#pragma unroll
            for (int k = 0; k < KH; ++k) {
                if constexpr (L) issue_lds(k, rn);
                else issue_reg(k, rn);
                __builtin_amdgcn_sched_barrier(0);
            }
            return nx;
        };

        // (two exits: the loop header is reached only from the register step,
        // so the wait counts the compiler derives there hold on every path)
        int64_t r = row0, r1 = row1;
        for (;;) {
            const int64_t r2 = step(std::integral_constant<bool, true>{}, r);
            r = r1;
            r1 = r2;
            if (r >= n) break;
            const int64_t r3 = step(std::integral_constant<bool, false>{}, r);
            r = r1;
            r1 = r3;
            if (r >= n) break;
        }
    }

    // ---- without the argmax, the ignored rows the leaders stepped over (all at
    // or past row G) are zeroed last, in chunks drawn from their own counter
    if constexpr (!ARGMAX) {
        const uint32_t row_bytes = static_cast<uint32_t>(nvec) * 16u;
        if (ctl0 && G < n) tagged_claim(ws_zero_chunks(a.workspace), tag);
        for (; G < n;) {
            if (ctl0) sh_chunk = tagged_draw(ws_zero_chunks(a.workspace), tag);
            __syncthreads();
            const int64_t c0 = static_cast<int64_t>(G) + static_cast<int64_t>(sh_chunk) * kHalfZeroChunk;
            if (c0 >= n) break;
            if (ctl) {
                const int64_t rr = c0 + (tid - ND);
                const bool ign = rr < n && !valid_label(a.labels[rr]);
                const unsigned long long msk = __ballot(ign);
                if (ctl0) sh_ign = msk;
            }
            __syncthreads();
            for (unsigned long long msk = sh_ign; msk; msk &= msk - 1) {
                const int64_t rz = c0 + __builtin_ctzll(msk);
                const __amdgpu_buffer_rsrc_t d = __builtin_amdgcn_make_buffer_rsrc(
                    static_cast<char *>(a.logits) + rz * a.ld * EL::bytes, 0, row_bytes, kBufferWord3);
                for (int k = 0; k * NT < nvec; ++k)
                    __builtin_amdgcn_raw_buffer_store_b128(zero4, d, voff + k * NT * 16, 0, kNonTemporal);
                if (tid == 0) store_through(a.loss_tok + rz, 0.0f);
            }
            __syncthreads();
        }
    }

    // ---- publish n_correct; the last workgroup folds the per-token losses and
    // these counts in a fixed order (as in ce_rows.h).  Losses come from the
    // control lane and, for zeroed rows, thread 0: both wait for theirs to land
    // before the ticket is taken.
    if (tid == 0) wait_vmem_all();
    __syncthreads();
    if (ctl0) {
        __hip_atomic_store(ws_correct(a.workspace) + blockIdx.x, correct, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_SYSTEM);
        wait_vmem_all();
        tagged_claim(ws_ticket(a.workspace), tag);
        const unsigned t = tagged_draw(ws_ticket(a.workspace), tag);
        sh_flag = t == static_cast<unsigned>(G) - 1u;
    }
    __syncthreads();
    if (!sh_flag) return;
    const long long n_valid = static_cast<long long>((static_cast<uint64_t>(sh_bc[7]) << 32) | sh_bc[6]);
    const long long n_bad = sh_nbad;
    double acc = 0.0;
    long long cor = __hip_atomic_load(ws_correct(a.workspace) + (tid < G ? tid : 0), __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_SYSTEM);
    constexpr int kFold = 8;
    for (int64_t r0 = 0; r0 < n; r0 += kFold * NT) {
        float lv[kFold];
#pragma unroll
        for (int u = 0; u < kFold; ++u) {
            const int64_t rr = r0 + u * NT + tid;
            lv[u] = __uint_as_float(__hip_atomic_load(reinterpret_cast<unsigned *>(a.loss_tok) + (rr < n ? rr : n - 1),
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

template <bool BF16, int KH, bool S, bool A, bool M>
hipError_t launch_half_variant(const CEArgs &a, int groups, hipStream_t st) {
    hipLaunchKernelGGL((ce_half_kernel<BF16, KH, S, A, M>), dim3(static_cast<unsigned>(groups)), dim3(NT), 0, st, a);
    return hipGetLastError();
}

template <bool BF16, int KH>
hipError_t launch_half_rows(const CEArgs &a, int groups, hipStream_t st) {
    const bool sc = a.softcap > 0.0f, am = a.argmax_out != nullptr, sm = a.eps != 0.0f;
#define LCE_HALF(S, A, M) return launch_half_variant<BF16, KH, S, A, M>(a, groups, st)
    if (sc) {
        if (am) { if (sm) LCE_HALF(true, true, true); else LCE_HALF(true, true, false); }
        else    { if (sm) LCE_HALF(true, false, true); else LCE_HALF(true, false, false); }
    } else {
        if (am) { if (sm) LCE_HALF(false, true, true); else LCE_HALF(false, true, false); }
        else    { if (sm) LCE_HALF(false, false, true); else LCE_HALF(false, false, false); }
    }
#undef LCE_HALF
}

}  // namespace dev
}  // namespace lce
