// gfx950 kernels of the Reverse All2All combine:
//   * signal_reset  -- zero signal slots in every slice before a launch;
//   * rev_a2a_pipelined -- persistent, role-split, tile-signalled combine;
//   * two_phase_exchange / two_phase_reorder -- the exchange-then-reorder variant.
//
// Combine ("Reverse All2All (EP MoE Distributed Kernel)", section "Reverse
// All2All Operator Semantics"): out_j[s, r*H + h, d] = in_r[j*S + s, h, d].
#include <type_traits>
#include <hip/hip_runtime.h>

#include "combine_geom.h"
#include "common.h"
#include "device.h"
#include "launch.h"
#include "queue.h"

namespace ra2a {

// ---------------------------------------------------------------------------
// Signal reset: slot i of every slice r (8 bytes at 128-byte spacing) := 0.
// ("Host Side Modifications": every signal is zeroed before each launch.)
__global__ void __launch_bounds__(kThreads) signal_reset_kernel(uint8_t* base, int64_t stride,
                                                                int W, int64_t sig_off,
                                                                int64_t nslots) {
    // thread k zeroes slot k in every slice (no index divisions)
    for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < nslots;
         k += (int64_t)gridDim.x * blockDim.x) {
        uint8_t* p = base + sig_off + k * (kSigStrideU64 * 8);
        for (int r = 0; r < W; ++r) *reinterpret_cast<uint64_t*>(p + r * stride) = 0ull;
    }
}

// Zero n contiguous 8-byte words (a kernel rather than a memset node, so that
// callers may capture it in a graph).
__global__ void __launch_bounds__(kThreads) zero_u64_kernel(uint64_t* p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0ull;
}

hipError_t launch_zero_u64(uint64_t* p, int64_t n, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    int64_t blocks = (n + kThreads - 1) / kThreads;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(zero_u64_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, st, p, n);
    return hipGetLastError();
}

hipError_t launch_signal_reset(uint8_t* base, int64_t stride, int W, int64_t sig_off,
                               int64_t nslots, hipStream_t st) {
    if (W <= 0 || nslots <= 0) return hipSuccess;
    int64_t blocks = (nslots + kThreads - 1) / kThreads;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(signal_reset_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, st, base,
                       stride, W, sig_off, nslots);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Copies vectors [lo, hi) of a row plan (combine_geom.h).  Thread t takes the
// vectors lo + t, lo + t + 256, ...; a cursor keeps their offsets without
// divisions.  Each round keeps U vectors per thread in flight (all loads issued
// before any store).  NTL / NTS: non-temporal loads / stores (data touched
// once: the input and the output), so that they do not displace the staging
// ring from the L2.
template <int V, int U, bool NTL, bool NTS>
__device__ __forceinline__ void copy_plan(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                          const RowPlan& p, int lo, int hi) {
    using T = typename Vec<V>::T;
    constexpr int kRound = U * kThreads;  // vectors per round
    const int vpr = p.run / V;
    // Rounds lying wholly inside [lo, hi) run without per-lane range tests (the
    // loop condition is uniform), so the compiler waits for each load just
    // before its store instead of draining every access before the first
    // store; one predicated round moves the tail.
    const int nfull = hi > lo ? (hi - lo) / kRound : 0;
    int idx = lo + (int)threadIdx.x;
    auto put = [](const T& v, uint8_t* d) {
        if (NTS)
            store_nt(v, reinterpret_cast<T*>(d));
        else
            *reinterpret_cast<T*>(d) = v;
    };
    auto get = [](const uint8_t* s) {
        const T* sp = reinterpret_cast<const T*>(s);
        return NTL ? load_nt(sp) : *sp;
    };
    if (p.B * p.C == 1 && lo == 0 && kThreads % vpr == 0) {
        // one run per row and whole rows per step: each step moves kThreads / vpr
        // rows down at the same column, so both offsets advance by constants
        const int rows = kThreads / vpr;
        const int row = idx / vpr, col = idx - row * vpr;
        const uint8_t* s0 = src + row * p.sa + (int64_t)col * V;
        uint8_t* d0 = dst + row * p.da + (int64_t)col * V;
        const int64_t ds = rows * p.sa, dd = rows * p.da;
        for (int k = 0; k < nfull; ++k) {
            T v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) v[u] = get(s0 + u * ds);
#pragma unroll
            for (int u = 0; u < U; ++u) put(v[u], d0 + u * dd);
            s0 += U * ds;
            d0 += U * dd;
        }
        idx += nfull * kRound;
        if (idx < hi) {
            T v[U];
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (idx + u * kThreads < hi) v[u] = get(s0 + u * ds);
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (idx + u * kThreads < hi) put(v[u], d0 + u * dd);
        }
        return;
    }
    PlanCursor c = cursor_start(p, V, vpr, (uint32_t)idx, kThreads);
    for (int k = 0; k < nfull; ++k) {
        T v[U];
        int64_t doff[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            v[u] = get(src + c.so);
            doff[u] = c.dofs;
            cursor_advance(c, p, vpr);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) put(v[u], dst + doff[u]);
    }
    idx += nfull * kRound;
    if (idx < hi) {
        T v[U];
        int64_t doff[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (idx + u * kThreads < hi) v[u] = get(src + c.so);
            doff[u] = c.dofs;
            cursor_advance(c, p, vpr);
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (idx + u * kThreads < hi) put(v[u], dst + doff[u]);
    }
}

// The same with device-scope write-through stores (kPolicyDevNt) through a
// buffer descriptor `dst` whose range covers the plan's destination (32-bit
// plan offsets): how the direct modes write out_j, so that a drain publishes
// the data device-wide (device.h).  Loads are non-temporal (the input is read
// once).
//
// `early(n)` runs once: right after the first full round's loads, with n = U of
// them the youngest memory operations in flight, or with n = 0 before the
// remainder when there is no full round.
struct NoEarly {
    template <class N>
    __device__ __forceinline__ void operator()(N) const {}
};

template <int V, int U, class Early = NoEarly>
__device__ __forceinline__ void copy_plan_wt(const uint8_t* __restrict__ src,
                                             __amdgpu_buffer_rsrc_t dst, const RowPlan& p, int lo,
                                             int hi, Early&& early = Early{}) {
    using T = typename Vec<V>::T;
    constexpr int kRound = U * kThreads;
    const int vpr = p.run / V;
    const int nfull = hi > lo ? (hi - lo) / kRound : 0;
    int idx = lo + (int)threadIdx.x;
    auto get = [](const uint8_t* s) { return load_nt(reinterpret_cast<const T*>(s)); };
    auto put = [&](const T& v, uint32_t off) { BufStore<V, kPolicyDevNt>::go(v, dst, off); };
    if (p.B * p.C == 1 && lo == 0 && kThreads % vpr == 0) {
        // whole rows per step: both offsets advance by constants
        const int rows = kThreads / vpr;
        const int row = idx / vpr, col = idx - row * vpr;
        const uint8_t* s0 = src + row * p.sa + (int64_t)col * V;
        uint32_t d0 = (uint32_t)(row * p.da + (int64_t)col * V);
        const int64_t ds = rows * p.sa;
        const uint32_t dd = (uint32_t)(rows * p.da);
        for (int k = 0; k < nfull; ++k) {
            T v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) v[u] = get(s0 + u * ds);
            if (k == 0) early(std::integral_constant<int, U>{});
#pragma unroll
            for (int u = 0; u < U; ++u) put(v[u], d0 + (uint32_t)u * dd);
            s0 += U * ds;
            d0 += (uint32_t)U * dd;
        }
        if (nfull == 0) early(std::integral_constant<int, 0>{});
        idx += nfull * kRound;
        if (idx < hi) {
            T v[U];
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (idx + u * kThreads < hi) v[u] = get(s0 + u * ds);
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (idx + u * kThreads < hi) put(v[u], d0 + (uint32_t)u * dd);
        }
        return;
    }
    PlanCursor c = cursor_start(p, V, vpr, (uint32_t)idx, kThreads);
    for (int k = 0; k < nfull; ++k) {
        T v[U];
        uint32_t doff[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            v[u] = get(src + c.so);
            doff[u] = (uint32_t)c.dofs;
            cursor_advance(c, p, vpr);
        }
        if (k == 0) early(std::integral_constant<int, U>{});
#pragma unroll
        for (int u = 0; u < U; ++u) put(v[u], doff[u]);
    }
    if (nfull == 0) early(std::integral_constant<int, 0>{});
    idx += nfull * kRound;
    if (idx < hi) {
        T v[U];
        uint32_t doff[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (idx + u * kThreads < hi) v[u] = get(src + c.so);
            doff[u] = (uint32_t)c.dofs;
            cursor_advance(c, p, vpr);
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (idx + u * kThreads < hi) put(v[u], doff[u]);
    }
}

// Copy of the runs (a, b) of a plan with C == 1 and sb == run, so that each a's
// B runs are one contiguous source range of B*run bytes: run (a, b) goes from
// src + a*sa + b*run to dst + a*da + b*db.  The ranges are moved in rounds of
// kThreads * V contiguous bytes (lane t takes bytes [t*V, t*V + V) of each), a
// after a, U rounds in flight (all loads, then all stores; a group may span
// several a); device-scope write-through stores as in copy_plan_wt.  The
// source offset of a round is the same for the whole workgroup (scalar
// registers) plus the lane's column.  The destination:
//  - runs of whole rounds: a round lies in one run, so its destination is also
//    workgroup-uniform plus the lane's column;
//  - any other run: each lane keeps its own (column in the run, destination),
//    advanced by the round's kThreads * V bytes with one wrap test per round.
// Each a's last, partial round (B*run not a multiple of the round) moves in a
// second pass, by the lanes whose bytes it holds.  Round offsets advance with
// selects, not branches, so that a group's loads issue back to back.  `late()`
// runs once, right after the loads of the last round group: a load it issues
// (a read of the reset flags) is younger than every copy load, so no store of
// the copy waits for it, and it completes under the last stores.
__device__ __forceinline__ bool run_shape_ok(const RowPlan& p) {
    return p.C == 1 && p.sb == p.run && p.run > 0;
}

template <int V, int U, typename Late>
__device__ __forceinline__ void copy_runs_wt(const uint8_t* __restrict__ src,
                                             __amdgpu_buffer_rsrc_t dst, const RowPlan& p,
                                             Late&& late) {
    using T = typename Vec<V>::T;
    constexpr int kChunk = kThreads * V;
    const uint32_t R = (uint32_t)p.run;
    const bool whole = R % kChunk == 0;              // runs of m whole rounds
    const int m = whole ? (int)(R / kChunk) : 1;     // rounds per run
    const int64_t len = (int64_t)p.B * R;            // bytes per a
    const int nq = (int)(len / kChunk);              // full rounds per a
    const uint32_t remb = (uint32_t)(len - (int64_t)nq * kChunk);  // bytes of a partial round
    const uint32_t lane = threadIdx.x * V;
    const uint32_t db = (uint32_t)p.db, da = (uint32_t)p.da;
    // other runs: the lane's column in its run and destination in round 0, and
    // the per-round steps (kThreads * V = sr runs + sc bytes)
    const uint32_t col0 = whole ? lane : lane % R;
    const uint32_t lane_dst = whole ? lane : (lane / R) * db + col0;
    const uint32_t sc = whole ? 0u : (uint32_t)kChunk % R;
    const uint32_t step = whole ? 0u : ((uint32_t)kChunk / R) * db + sc;
    // whole runs: destination steps to the next round of the same run, to the
    // next run of the same a, and from an a's last round to the next a's first
    // (modulo 2^32, like the offsets)
    const uint32_t next_run = db - (uint32_t)(m - 1) * kChunk;
    const uint32_t next_a = da - ((uint32_t)(p.B - 1) * db + (uint32_t)(m - 1) * kChunk);
    const int64_t src_next_a = p.sa - (int64_t)(nq - 1) * kChunk;
    const int total = p.A * nq;
    const uint8_t* const s_lane = src + lane;
    int q = 0, c = 0;
    int64_t so = 0;
    uint32_t dof = lane_dst;  // whole runs: the destination; others: relative to abase
    uint32_t abase = 0, col = col0;
    auto advance = [&](auto whole_c) {
        constexpr bool WHOLE = decltype(whole_c)::value;
        const bool end_a = q + 1 == nq;
        so += end_a ? src_next_a : (int64_t)kChunk;
        if (WHOLE) {
            const bool end_run = c + 1 == m;
            dof += end_a ? next_a : (end_run ? next_run : (uint32_t)kChunk);
            c = end_run ? 0 : c + 1;
        } else {
            col += sc;
            dof += step;
            const bool wrap = col >= R;
            col = wrap ? col - R : col;
            dof = wrap ? dof + (db - R) : dof;
            col = end_a ? col0 : col;
            dof = end_a ? lane_dst : dof;
            abase = end_a ? abase + da : abase;
        }
        q = end_a ? 0 : q + 1;
    };
    int f = 0;
    auto group = [&](auto kc, auto whole_c) {
        constexpr int K = decltype(kc)::value;
        int64_t sofs[K];
        uint32_t d[K];
#pragma unroll
        for (int u = 0; u < K; ++u) {
            sofs[u] = so;
            d[u] = abase + dof;
            advance(whole_c);
        }
        T v[K];
#pragma unroll
        for (int u = 0; u < K; ++u) v[u] = load_nt(reinterpret_cast<const T*>(s_lane + sofs[u]));
        if (f + K == total) late();
#pragma unroll
        for (int u = 0; u < K; ++u) BufStore<V, kPolicyDevNt>::go(v[u], dst, d[u]);
        f += K;
    };
    auto rounds = [&](auto whole_c) {
        while (f + U <= total) group(std::integral_constant<int, U>{}, whole_c);
        if (U >= 4 && f + U / 2 <= total)
            group(std::integral_constant<int, (U >= 4 ? U / 2 : 1)>{}, whole_c);
        while (f < total) group(std::integral_constant<int, 1>{}, whole_c);
    };
    if (whole)
        rounds(std::true_type{});
    else
        rounds(std::false_type{});
    if (total == 0) late();
    // the partial rounds, one per a: bytes nq*kChunk + lane of each a's range
    if (remb > 0 && lane < remb) {
        const uint32_t o = (uint32_t)nq * kChunk + lane;
        const uint32_t ri = o / R;
        const int64_t s_part = (int64_t)nq * kChunk;
        const uint32_t d_part = ri * db + (o - ri * R);
        int a0 = 0;
        auto part = [&](auto kc) {
            constexpr int K = decltype(kc)::value;
            T v[K];
#pragma unroll
            for (int u = 0; u < K; ++u)
                v[u] = load_nt(reinterpret_cast<const T*>(s_lane + (int64_t)(a0 + u) * p.sa + s_part));
#pragma unroll
            for (int u = 0; u < K; ++u)
                BufStore<V, kPolicyDevNt>::go(v[u], dst, (uint32_t)(a0 + u) * da + d_part);
            a0 += K;
        };
        while (a0 + U <= p.A) part(std::integral_constant<int, U>{});
        while (a0 < p.A) part(std::integral_constant<int, 1>{});
    }
}

// The mirror image of copy_runs_wt, for the dispatch's row units: each a's B
// runs are one contiguous destination range (db == run) at dst + a*da (another
// slice for every a, so each round takes its own descriptor), and the source
// holds them at src + a*sa + b*sb.  Rounds walk the destination range; the
// source offset is workgroup-uniform for runs of whole rounds, else tracked per
// lane as copy_runs_wt tracks its destination.
template <int V, int U, typename Late>
__device__ __forceinline__ void copy_runs_inv_wt(const uint8_t* __restrict__ src, uint8_t* dst,
                                                 const RowPlan& p, Late&& late) {
    using T = typename Vec<V>::T;
    constexpr int kChunk = kThreads * V;
    const uint32_t R = (uint32_t)p.run;
    const bool whole = R % kChunk == 0;
    const int m = whole ? (int)(R / kChunk) : 1;
    const int64_t len = (int64_t)p.B * R;            // bytes per a (its destination range)
    const int nq = (int)(len / kChunk);
    const uint32_t remb = (uint32_t)(len - (int64_t)nq * kChunk);
    const uint32_t lane = threadIdx.x * V;
    const uint32_t sb = (uint32_t)p.sb, sa = (uint32_t)p.sa;
    const uint32_t col0 = whole ? lane : lane % R;
    const uint32_t lane_src = whole ? lane : (lane / R) * sb + col0;
    const uint32_t sc = whole ? 0u : (uint32_t)kChunk % R;
    const uint32_t step = whole ? 0u : ((uint32_t)kChunk / R) * sb + sc;
    const uint32_t next_run = sb - (uint32_t)(m - 1) * kChunk;
    const uint32_t next_a = sa - ((uint32_t)(p.B - 1) * sb + (uint32_t)(m - 1) * kChunk);
    const uint32_t span = (uint32_t)len;
    const int total = p.A * nq;
    int q = 0, c = 0, a0 = 0;
    uint32_t sof = lane_src, abase = 0, col = col0;
    auto advance = [&](auto whole_c) {
        constexpr bool WHOLE = decltype(whole_c)::value;
        const bool end_a = q + 1 == nq;
        if (WHOLE) {
            const bool end_run = c + 1 == m;
            sof += end_a ? next_a : (end_run ? next_run : (uint32_t)kChunk);
            c = end_run ? 0 : c + 1;
        } else {
            col += sc;
            sof += step;
            const bool wrap = col >= R;
            col = wrap ? col - R : col;
            sof = wrap ? sof + (sb - R) : sof;
            col = end_a ? col0 : col;
            sof = end_a ? lane_src : sof;
            abase = end_a ? abase + sa : abase;
        }
        a0 = end_a ? a0 + 1 : a0;
        q = end_a ? 0 : q + 1;
    };
    int f = 0;
    auto group = [&](auto kc, auto whole_c) {
        constexpr int K = decltype(kc)::value;
        uint32_t s_off[K], d_off[K];
        int a_u[K];
#pragma unroll
        for (int u = 0; u < K; ++u) {
            s_off[u] = abase + sof;
            d_off[u] = (uint32_t)q * kChunk + lane;
            a_u[u] = a0;
            advance(whole_c);
        }
        T v[K];
#pragma unroll
        for (int u = 0; u < K; ++u) v[u] = load_nt(reinterpret_cast<const T*>(src + s_off[u]));
        if (f + K == total) late();
#pragma unroll
        for (int u = 0; u < K; ++u)
            BufStore<V, kPolicyDevNt>::go(v[u], make_rsrc_uniform(dst + (int64_t)a_u[u] * p.da, span),
                                          d_off[u]);
        f += K;
    };
    auto rounds = [&](auto whole_c) {
        while (f + U <= total) group(std::integral_constant<int, U>{}, whole_c);
        if (U >= 4 && f + U / 2 <= total)
            group(std::integral_constant<int, (U >= 4 ? U / 2 : 1)>{}, whole_c);
        while (f < total) group(std::integral_constant<int, 1>{}, whole_c);
    };
    if (whole)
        rounds(std::true_type{});
    else
        rounds(std::false_type{});
    if (total == 0) late();
    // the partial rounds, one per a: bytes nq*kChunk + lane of each destination range
    if (remb > 0 && lane < remb) {
        const uint32_t o = (uint32_t)nq * kChunk + lane;
        const uint32_t ri = o / R;
        const uint32_t s_part = ri * sb + (o - ri * R);
        for (int a1 = 0; a1 < p.A; ++a1) {
            const T v = load_nt(reinterpret_cast<const T*>(src + (uint32_t)a1 * sa + s_part));
            BufStore<V, kPolicyDevNt>::go(v, make_rsrc_uniform(dst + (int64_t)a1 * p.da, span), o);
        }
    }
}

// The same, reading the source through a buffer descriptor with cache policy
// POLICY at 32-bit offsets src_off + (plan offset).
template <int V, int U, int POLICY, bool NTS>
__device__ __forceinline__ void copy_plan_buf(__amdgpu_buffer_rsrc_t src, uint32_t src_off,
                                              uint8_t* __restrict__ dst, const RowPlan& p, int lo,
                                              int hi) {
    using T = typename Vec<V>::T;
    constexpr int kRound = U * kThreads;
    const int vpr = p.run / V;
    const int nfull = hi > lo ? (hi - lo) / kRound : 0;
    int idx = lo + (int)threadIdx.x;
    auto put = [](const T& v, uint8_t* d) {
        if (NTS)
            store_nt(v, reinterpret_cast<T*>(d));
        else
            *reinterpret_cast<T*>(d) = v;
    };
    PlanCursor c = cursor_start(p, V, vpr, (uint32_t)idx, kThreads);
    for (int k = 0; k < nfull; ++k) {  // whole rounds: no per-lane tests
        T v[U];
        int64_t doff[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            v[u] = BufLoad<V, POLICY>::go(src, src_off + (uint32_t)c.so);
            doff[u] = c.dofs;
            cursor_advance(c, p, vpr);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) put(v[u], dst + doff[u]);
    }
    idx += nfull * kRound;
    if (idx < hi) {
        T v[U];
        int64_t doff[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (idx + u * kThreads < hi) v[u] = BufLoad<V, POLICY>::go(src, src_off + (uint32_t)c.so);
            doff[u] = c.dofs;
            cursor_advance(c, p, vpr);
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (idx + u * kThreads < hi) put(v[u], dst + doff[u]);
    }
}

// ---------------------------------------------------------------------------
// The signal-pipelined persistent combine.
//
// Work is organised in tile streams: stream (j, merged head block, d block) is
// the sequence of S-blocks b = 0 .. nbs-1 of destination j.  A producer piece
// is one source r's part of a tile (stream, S-block).
//
// Direct mode (the default, direct_path below): producers store each piece into
// its final place in out_j and signal it; nothing waits, the schedule is static.
//
// Staged mode: the streams are cut into NG contiguous groups, one per XCD.  Each
// group has a work queue (combine_geom.h: group_queue / task_of) holding its
// producer pieces and consumer work items (parts of a tile's unit) in an order
// in which every wait points backwards.  Workgroups claim queue positions one
// at a time with an atomic counter and run each task to completion, so the
// earliest unfinished task can always proceed: no deadlock, whatever the
// number of resident workgroups, and an ordinary launch suffices.
//
// Placement (staged mode, SYNC == kSyncXcd).  A group's tasks must all run on
// one XCD, so that producers and consumers meet in that XCD's L2 and
// synchronise with the XCD-local sequences of device.h instead of device-wide
// L2 write-backs and invalidations.  A workgroup reads the XCD it runs on from
// the XCC_ID register and claims from its own XCD's group; once that queue is
// drained it may take over a group whose home XCD has not claimed anything (a
// group whose XCD received no workgroup, or received them late), and then only
// workgroups of the taking XCD serve it.  So every group is served, by one XCD,
// whatever the dispatcher does.  SYNC == kSyncAgent uses device-wide
// release/acquire and lets every workgroup help every group.
//
// Staged producer piece: wait until ring slot b mod R of its stream has been
// handed back by the consumers of S-block b - R (credit count; never when the
// ring is not reused), copy in_r -> staging_j, release, then wave 0 signals the
// piece's signal tiles (SET 1 on the piece's slot, or ADD 1 on the tile's slot).
//
// Staged consumer item: wait until each of its signal tiles reads W (ADD) or 1
// (SET), copy its part of the unit staging_j -> out_j, release, add 1 to the
// slot's hand-back count, optionally stamp the completion time.
//
// Every wait is also bounded in time (spin_until).
// A piece's waits before its copy starts: for the hand-back of its ring slot
// (staged mode, ring reused) and as a delayed (straggler) source.  False if a
// bounded wait gave up.
__device__ __forceinline__ bool piece_wait(const PipeArgs& a, const Piece& p, int* lds_flag) {
    if (p.b >= a.R &&
        !group_wait<false>(reinterpret_cast<const uint64_t*>(a.base + p.credit), kCmpGe,
                           p.credit_need, a.timeout, a.err, lds_flag))
        return false;
    if (p.r == a.straggler && a.delay) {
        // a busy wait of n0 + u ticks of the 100 MHz device clock, u uniform in
        // [0, n0] from SplitMix64 indexed by the piece
        if (threadIdx.x == 0) {
            const uint64_t id =
                ((((uint64_t)p.b * (uint64_t)a.nstreams + p.sid) * (uint64_t)a.nsub + p.sub) * a.W) + p.r;
            const uint64_t n = a.delay + splitmix64(a.seed, id) % ((uint64_t)a.delay + 1ull);
            const uint64_t t0 = rtc_now();
            while (rtc_now() - t0 < n) __builtin_amdgcn_s_sleep(1);
        }
        __syncthreads();
    }
    return true;
}

// Wave 0 signals the signal tiles of a piece (after the release).
__device__ __forceinline__ void piece_signal(const PipeArgs& a, int64_t sig, int64_t step, int n) {
    const int op = a.protocol == kSigAdd ? kSigAdd : kSigSet;
    for (int k = threadIdx.x; k < n && threadIdx.x < 64; k += 64)
        sig_update(reinterpret_cast<uint64_t*>(a.base + sig + k * step), 1ull, op);
}

// Staged mode, producer piece: wait for the ring slot's hand-back, copy in_r ->
// staging_j (plain stores: the consumers read it back from this XCD's L2),
// release, signal.
template <int V, int SYNC>
__device__ __forceinline__ bool run_piece(const PipeArgs& a, int g, int64_t pc, int* lds_flag) {
    const Piece p = piece_of(a, g, pc);
    if (!piece_wait(a, p, lds_flag)) return false;
    copy_plan<V, 8, true, false>(a.base + p.src, a.base + p.dst, p.pl, 0, plan_vectors(p.pl, V));
    group_release<SYNC>();
    piece_signal(a, p.sig, p.sig_step, p.nsig);
    return true;
}

// Staged mode, consumer item: wait for the unit's signal tiles, copy its part
// staging_j -> out_j, release, hand the slot back.
template <int V, int SYNC>
__device__ __forceinline__ bool run_item(const PipeArgs& a, int g, int64_t it, int* lds_flag) {
    uint8_t* const base = a.base;
    const Item q = item_of(a, g, it, V);
    // XCD-local: staging is read with device-scope (L1-bypassing) loads from the
    // L2 this XCD's producers wrote it into, so no invalidation is needed.
    // Device-wide: the acquire drops stale L1 and L2 lines first.
    if (!group_wait_all<SYNC == kSyncAgent>(reinterpret_cast<const uint64_t*>(base + q.sig),
                                            q.sig_step, q.nsig, kCmpEq, q.sig_want, a.timeout,
                                            a.err, lds_flag))
        return false;
    if (q.hi > q.lo) {
        if (SYNC == kSyncXcd) {
            // the staging slice: the destination's, or (pull) the sender's
            const int64_t stg = (int64_t)(a.pull ? q.r0 : q.j) * a.stride + a.stg_off;
            copy_plan_buf<V, 8, kPolicySc1, true>(make_rsrc_uniform(base + stg, (uint32_t)a.ring_bytes),
                                                  (uint32_t)(q.src - stg), base + q.dst, q.pl, q.lo,
                                                  q.hi);
        } else {
            copy_plan<V, 8, false, true>(base + q.src, base + q.dst, q.pl, q.lo, q.hi);
        }
    }
    group_release<SYNC>();
    if (threadIdx.x == 0 && !a.bulk)  // the bulk mode has no ring to hand back
        sig_update(reinterpret_cast<uint64_t*>(base + q.credit), 1ull, kSigAdd);
    if (a.stamps && threadIdx.x < 64) {
        const uint64_t now = rtc_now();
        for (int k = threadIdx.x; k < q.nsig; k += 64)
            __hip_atomic_fetch_max(a.stamps + (int64_t)q.j * a.units_per_dest + q.unit_index +
                                       k * q.unit_step,
                                   now, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return true;
}

// In-launch signal reset (direct mode; "Host Side Modifications": every signal
// is zero before any producer of a launch signals).  Zeroing workgroup k
// clears slots [k * reset_chunk, (k + 1) * reset_chunk) of every slice and its
// share of the timestamps, releases device-wide (every wave's stores reach the
// device-wide coherence point), then sets reset flag k to this launch's tag.
// It waits on nothing, so it always finishes.
__device__ __forceinline__ void reset_share(const PipeArgs& a, int k) {
    const int64_t lo = (int64_t)k * a.reset_chunk;
    const int64_t hi = geom_min(lo + a.reset_chunk, a.reset_slots);
    for (int64_t i = lo + threadIdx.x; i < hi; i += kThreads) {
        uint8_t* p = a.base + a.sig_off + i * (kSigStrideU64 * 8);
        for (int r = 0; r < a.W; ++r) *reinterpret_cast<uint64_t*>(p + r * a.stride) = 0ull;
    }
    if (a.stamps) {
        const int64_t n = (int64_t)a.W * a.units_per_dest;
        const int64_t slo = (int64_t)k * a.stamp_chunk;
        const int64_t shi = geom_min(slo + a.stamp_chunk, n);
        for (int64_t i = slo + threadIdx.x; i < shi; i += kThreads) a.stamps[i] = 0ull;
    }
    wg_release();
    if (threadIdx.x == 0)
        __hip_atomic_store(reinterpret_cast<uint64_t*>(a.base + a.flag_off) + (int64_t)k * kSigStrideU64,
                           a.reset_tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ const uint64_t* reset_flag(const PipeArgs& a, int k) {
    return reinterpret_cast<const uint64_t*>(a.base + a.flag_off) + (int64_t)k * kSigStrideU64;
}

// Before a workgroup's first signal: every reset flag carries this launch's tag
// (lane k of wave 0 polls flag k; `early`, lane k's earlier read of it, spares
// the poll when it already held the tag), then wave 0 -- the one that signals
// and stamps -- acquires.  False, uniformly, if a bounded wait gave up.
__device__ __forceinline__ bool reset_published(const PipeArgs& a, uint64_t early = 0ull) {
    bool ok = true;
    if ((int)threadIdx.x < a.reset_nz && early != a.reset_tag)
        ok = spin_until(reset_flag(a, (int)threadIdx.x), kCmpEq, a.reset_tag, a.timeout, a.err);
    if (threadIdx.x < 64) fence_acquire_agent();
    return __syncthreads_and(ok ? 1 : 0) != 0;
}

// Work distribution of the direct modes.  Persistent workgroup k first takes
// piece (or row unit) k.  With a static schedule (dyn == 0) it then takes k +
// piece_grid, k + 2 piece_grid, ...; with dyn == 1 each further one is claimed
// from a counter in the spare queue word (zeroed by the reset, so the first
// claim waits until the reset is published), issued when the previous piece
// starts so that the claim's round trip hides under its copy.  Claimed work
// stays balanced when pieces are many and their speed varies with where in
// HBM they lie.
struct Claimer {
    uint64_t* ctr;
    int64_t grid;
    int64_t next;   // lane 0: the claimed piece, or -1 if none is claimed yet
};

__device__ __forceinline__ Claimer claimer(const PipeArgs& a) {
    Claimer c;
    c.ctr = reinterpret_cast<uint64_t*>(a.base + a.claim_off);
    c.grid = a.piece_grid;
    c.next = -1;
    return c;
}

// Lane 0 claims the piece after the current one (dynamic schedule, once the
// reset is published).
__device__ __forceinline__ void claim_ahead(const PipeArgs& a, Claimer& c, bool published) {
    if (a.dyn && published && threadIdx.x == 0 && c.next < 0)
        c.next = c.grid + (int64_t)__hip_atomic_fetch_add(c.ctr, 1ull, __ATOMIC_RELAXED,
                                                          __HIP_MEMORY_SCOPE_AGENT);
}

// The workgroup's next piece (uniform across it).
__device__ __forceinline__ int64_t next_piece(const PipeArgs& a, Claimer& c, int64_t cur,
                                              int64_t* lds_next) {
    if (!a.dyn) return cur + c.grid;
    if (threadIdx.x == 0) *lds_next = c.next;
    c.next = -1;
    __syncthreads();
    const int64_t n = *lds_next;
    __syncthreads();
    return n;
}

// Wave 0: completion stamps (the device clock) of n signal tiles `step` slots apart.
__device__ __forceinline__ void stamp_tiles(const PipeArgs& a, int j, int64_t first, int64_t step,
                                            int n) {
    if (a.stamps && threadIdx.x < 64) {
        const uint64_t now = rtc_now();
        for (int k = threadIdx.x; k < n; k += 64)
            __hip_atomic_fetch_max(a.stamps + (int64_t)j * a.units_per_dest + first + k * step, now,
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Lane 0 adds 1 to an arrival counter; true (uniformly) for the arrival that
// brings it to `need`.
__device__ __forceinline__ bool arrive(const PipeArgs& a, int64_t cnt, uint64_t need, int* lds_flag) {
    if (threadIdx.x == 0) {
        const uint64_t before = __hip_atomic_fetch_add(reinterpret_cast<uint64_t*>(a.base + cnt), 1ull,
                                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *lds_flag = before + 1ull == need ? 1 : 0;
    }
    __syncthreads();
    const bool last = *lds_flag != 0;
    __syncthreads();
    return last;
}

// Direct mode, per-source pieces.  Producers store straight into out_j, so no
// consumer has data to move.  A piece covers part `sub` of the tile's rows for
// one source.  With one part per tile (nsub == 1) the piece signals its tiles
// itself: ADD 1 (the tile is complete at W) or SET 1 on its (tile, source)
// slot.  With several, each piece adds 1 to its tile's arrival counter (per
// source under SET) and the piece that completes it signals as all W (or the
// source's) pieces would have: ADD W, or SET 1.  Stores are device-scope
// write-through (copy_plan_wt), so a drain and a barrier publish them on every
// XCD before the signal or the count (the drain of one piece's stores is the wait
// for the next piece's first loads); the piece that reads the counter's last
// arrival follows every other piece's drained stores.  The optional completion
// stamp of a tile is the latest of its signalling pieces' stamps.  The only
// wait is for the in-launch reset's flags.  The reset runs on the reset_nz
// workgroups with the lowest block ids.  Those are dispatched first --
// workgroups of one launch are dispatched in id order -- so they hold their
// compute-unit slots before any workgroup that waits for them exists, whatever
// else occupies the device; they wait on nothing, so the wait always ends.
template <int V, int SYNC>
__device__ __forceinline__ void direct_path(const PipeArgs& a, int* lds_flag) {
    __shared__ int64_t lds_next;
    const int nz = a.reset_nz;
    if ((int)blockIdx.x < nz) {  // a zeroing workgroup of the in-launch reset
        reset_share(a, (int)blockIdx.x);
        return;
    }
    bool published = a.reset_tag == 0ull;
    const int64_t total = total_pieces(a);
    const int op = a.protocol == kSigAdd ? kSigAdd : kSigSet;
    const uint64_t done_val = a.protocol == kSigAdd ? (uint64_t)a.W : 1ull;
    const int64_t step = slot_step(a);
    Claimer cl = claimer(a);
    // The piece whose stores are issued but not yet published (`pend`): its signal,
    // or its arrival, goes out once those stores have drained -- right after the
    // next piece's first loads, whose wait then covers them (vector memory
    // operations complete in issue order), or at the end.  So no workgroup sits in a
    // drain between two pieces with nothing in flight.
    bool pend = false;
    Piece q{};
    // wave 0, once every wave's stores of q have drained
    auto publish = [&]() {
        if (a.nsub == 1) {
            piece_signal(a, q.sig, q.sig_step, q.nsig);
            stamp_tiles(a, q.j, q.unit_index, step, q.nsig);
        } else if (threadIdx.x < 64) {
            uint64_t before = 0ull;
            if (threadIdx.x == 0)
                before = __hip_atomic_fetch_add(reinterpret_cast<uint64_t*>(a.base + q.cnt), 1ull,
                                                __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)before);
            const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(before >> 32));
            if ((((uint64_t)hi << 32) | lo) + 1ull == q.cnt_need) {
                for (int k = threadIdx.x; k < q.nsig; k += 64)
                    sig_update(reinterpret_cast<uint64_t*>(a.base + q.sig + k * q.sig_step), done_val, op);
                stamp_tiles(a, q.j, q.unit_index, step, q.nsig);
            }
        }
    };
    for (int64_t gp = (int)blockIdx.x - nz; gp < total;) {
        claim_ahead(a, cl, published);
        const Piece p = direct_piece(a, gp);
        // a delayed (straggler) piece waits before its copy: publish the pending
        // piece first, so that its tiles are not held up by the delay
        if (pend && p.r == a.straggler && a.delay) {
            group_release_written_through();
            publish();
            pend = false;
        }
        if (!piece_wait(a, p, lds_flag)) return;
        auto early = [&](auto n) {
            if (pend) {
                asm volatile("s_waitcnt vmcnt(%0)" ::"i"(decltype(n)::value) : "memory");
                __syncthreads();  // every wave's stores of q have drained
                publish();
                pend = false;
            }
        };
        // final place: device-scope write-through stores, so a drain publishes them
        copy_plan_wt<V, 8>(a.base + p.src, make_rsrc_uniform(a.base + p.dst, plan_span(p.pl)), p.pl,
                           0, plan_vectors(p.pl, V), early);
        if (!published) {  // before any signal (the first is the next piece's)
            if (!reset_published(a)) return;
            published = true;
            claim_ahead(a, cl, published);
        }
        q = p;
        pend = true;
        gp = next_piece(a, cl, gp, &lds_next);
    }
    if (pend) {
        group_release_written_through();
        publish();
    }
}

// Direct mode with row units (RA2A_MODE_ROWS; combine_geom.h row_unit).  A
// unit copies its rows of every source into out_j with device-scope
// write-through stores (the destination one contiguous range), drains them, and
// adds 1 to the S-block's arrival counter.  Under ADD, when W is a multiple of
// the block's unit count nub, each unit also adds W / nub to every signal tile
// of the block, after its own drain: a tile reaches W exactly when all nub units
// have stored.  Otherwise the unit that completes the block's count marks every
// signal tile of the block complete: every other unit of the block drained its
// stores before its add, and the completing unit read the counter after all of
// them, so the block's rows are performed device-wide before these signals.
// Counter and signals are zeroed by the in-launch reset, so both wait for its
// flags.  Work is distributed as in direct_path.
template <int V>
__device__ __forceinline__ void rows_path(const PipeArgs& a, int* lds_flag) {
    __shared__ int64_t lds_next;
    const int nz = a.reset_nz;
    if ((int)blockIdx.x < nz) {  // a zeroing workgroup of the in-launch reset
        reset_share(a, (int)blockIdx.x);
        return;
    }
    const bool add = a.protocol == kSigAdd;
    const int op = add ? kSigAdd : kSigSet;
    const uint64_t val = add ? (uint64_t)a.W : 1ull;
    bool published = a.reset_tag == 0ull;
    Claimer cl = claimer(a);
    for (int64_t u = (int)blockIdx.x - nz; u < a.nunits;) {
        claim_ahead(a, cl, published);
        const RowUnit q = row_unit(a, u);
        // (the combine's destination: one slice, one descriptor)
        const __amdgpu_buffer_rsrc_t dst =
            make_rsrc_uniform(a.base + q.dst, a.inverse ? 0u : plan_span(q.pl));
        // Until the reset is known to be published, lane k < nz of wave 0 reads
        // reset flag k at the end of the copy, behind its last loads (a read in
        // the middle held up the next round's stores, which wait in order behind
        // it); the check after the drain then has nothing left to wait for unless
        // that read came too early.
        uint64_t early = 0ull;
        auto poll = [&]() {
            if (!published && (int)threadIdx.x < nz) early = sig_load(reset_flag(a, (int)threadIdx.x));
        };
        if (a.inverse) {
            if (a.ru == 4)
                copy_runs_inv_wt<V, 4>(a.base + q.src, a.base + q.dst, q.pl, poll);
            else
                copy_runs_inv_wt<V, 8>(a.base + q.src, a.base + q.dst, q.pl, poll);
        } else if (run_shape_ok(q.pl)) {
            if (a.ru == 4)
                copy_runs_wt<V, 4>(a.base + q.src, dst, q.pl, poll);
            else
                copy_runs_wt<V, 8>(a.base + q.src, dst, q.pl, poll);
        } else {
            poll();
            copy_plan_wt<V, 8>(a.base + q.src, dst, q.pl, 0, plan_vectors(q.pl, V));
        }
        group_release_written_through();
        if (!published) {
            if (!reset_published(a, early)) return;
            published = true;
            claim_ahead(a, cl, published);
        }
        // ADD protocol with W a multiple of the block's unit count: every unit
        // adds its share W / nub to each tile of the block (a tile reaches W once
        // all of them have stored their rows) and counts itself, with nothing to
        // wait for.  Otherwise the unit that completes the count signals for all.
        const uint64_t share = add && a.W % q.nub == 0 ? (uint64_t)(a.W / q.nub) : 0ull;
        // (the dispatch signals every destination's slice: nd = W, one slice apart)
        const int nall = q.nd * q.nsig;
        auto signal_all = [&](uint64_t v, int sop) {
            for (int i = threadIdx.x; i < nall; i += 64) {
                const int d = i / q.nsig, k = i - d * q.nsig;
                sig_update(reinterpret_cast<uint64_t*>(a.base + q.sig + (int64_t)d * a.stride +
                                                       (int64_t)k * q.sig_step),
                           v, sop);
            }
            for (int d = 0; d < q.nd; ++d)
                stamp_tiles(a, q.nd == 1 ? q.j : d, q.unit_index, q.unit_step, q.nsig);
        };
        if (share != 0ull) {
            if (threadIdx.x < 64) {
                if (threadIdx.x == 0) sig_update(reinterpret_cast<uint64_t*>(a.base + q.cnt), 1ull, kSigAdd);
                signal_all(share, kSigAdd);
            }
        } else if (arrive(a, q.cnt, (uint64_t)q.nub, lds_flag) && threadIdx.x < 64) {
            signal_all(val, op);
        }
        u = next_piece(a, cl, u, &lds_next);
    }
}

template <int V, int SYNC, bool DIRECT>
__global__ void __launch_bounds__(kThreads) rev_a2a_pipelined_kernel(PipeArgs a) {
    __shared__ int lds_flag;
    __shared__ int64_t lds_pos[2];
    if (DIRECT) {
        if (a.rows)
            rows_path<V>(a, &lds_flag);
        else
            direct_path<V, SYNC>(a, &lds_flag);
        return;
    }
    // Staged mode.  XCD-local sync binds each group to one XCD (queue.h); with
    // device-wide sync any workgroup serves any group, its home group first.
    constexpr bool kOwned = SYNC == kSyncXcd;
    // queue words: slice 0, after the hand-back counters
    uint64_t* const qw = reinterpret_cast<uint64_t*>(a.base + a.sig_off) +
                         (a.regionA + a.regionB) * kSigStrideU64;
    const uint32_t xcc = xcc_id();
    const int home = SYNC == kSyncXcd ? (int)(xcc % (uint32_t)a.NG) : (int)(blockIdx.x % a.NG);
    QueueClaim qc;  // thread 0's
    int k = 0;
    for (int gi = 0; gi < a.NG; ++gi) {
        const int g = (home + gi) % a.NG;
        if (threadIdx.x == 0) lds_pos[k & 1] = queue_first<kOwned>(qw, g, gi, xcc, qc);
        __syncthreads();
        // positions are wave-uniform: keep them (and all task geometry) scalar
        int64_t pos = (int64_t)__builtin_amdgcn_readfirstlane((int)lds_pos[k & 1]);
        ++k;
        if (pos < 0) continue;
        const GroupQueue Q = group_queue(a, g);
        while (true) {
            if (pos >= Q.total) {
                if (threadIdx.x == 0) queue_drained(qw, g, pos, Q.total, qc);
                break;
            }
            // claim the next position while this task runs (positions a workgroup
            // claims increase, so it still runs its tasks in queue order)
            uint64_t nxt = 0;
            if (threadIdx.x == 0) nxt = queue_next(qc);
            int64_t idx = 0;
            const bool ok = task_of(Q, pos, &idx) ? run_piece<V, SYNC>(a, g, idx, &lds_flag)
                                                  : run_item<V, SYNC>(a, g, idx, &lds_flag);
            if (!ok) return;  // a wait gave up: the error word is raised, everyone leaves
            if (threadIdx.x == 0) lds_pos[k & 1] = (int64_t)nxt;
            __syncthreads();
            pos = (int64_t)__builtin_amdgcn_readfirstlane((int)lds_pos[k & 1]);
            ++k;
        }
    }
}

template <int V, int SYNC, bool DIRECT>
static const void* pipelined_fn() {
    return reinterpret_cast<const void*>(&rev_a2a_pipelined_kernel<V, SYNC, DIRECT>);
}

template <int SYNC, bool DIRECT>
static const void* pipelined_fn_v(int V) {
    switch (V) {
        case 16: return pipelined_fn<16, SYNC, DIRECT>();
        case 8: return pipelined_fn<8, SYNC, DIRECT>();
        case 4: return pipelined_fn<4, SYNC, DIRECT>();
        case 2: return pipelined_fn<2, SYNC, DIRECT>();
        default: return pipelined_fn<1, SYNC, DIRECT>();
    }
}

static const void* pipelined_kernel(int V, int sync, int direct) {
    if (direct)
        return sync == kSyncXcd ? pipelined_fn_v<kSyncXcd, true>(V) : pipelined_fn_v<kSyncAgent, true>(V);
    return sync == kSyncXcd ? pipelined_fn_v<kSyncXcd, false>(V) : pipelined_fn_v<kSyncAgent, false>(V);
}

// The work queues make the kernel deadlock-free at any residency: an ordinary launch.
hipError_t launch_pipelined(const PipeArgs& a, int V, int grid, hipStream_t st) {
    void* args[] = {const_cast<PipeArgs*>(&a)};
    return hipLaunchKernel(pipelined_kernel(V, a.sync, a.direct), dim3(grid), dim3(kThreads), args, 0,
                           st);
}

hipError_t pipelined_blocks_per_cu(int V, int sync, int direct, int* n) {
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(n, pipelined_kernel(V, sync, direct), kThreads,
                                                        0);
}

// ---------------------------------------------------------------------------
// Placement probe: the XCD each workgroup of a launch runs on.
__global__ void xcc_probe_kernel(uint32_t* out, int n) {
    if (threadIdx.x == 0 && (int)blockIdx.x < n) out[blockIdx.x] = xcc_id();
}

hipError_t launch_xcc_probe(uint32_t* out, int n, hipStream_t st) {
    hipLaunchKernelGGL(xcc_probe_kernel, dim3(n), dim3(64), 0, st, out, n);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Two-phase variant ("UDMA Optimized Implementation", "Two-Phase Data Copy").
// Phase 1: segment (r -> j): in_r rows [j*S, (j+1)*S) (contiguous S*H*D
// elements) -> slot r of staging_j, laid out [W][S][H][D].
template <int V>
__global__ void __launch_bounds__(kThreads) two_phase_exchange_kernel(TwoPhaseArgs a) {
    const int seg = blockIdx.y;  // r * W + j
    const int r = seg / a.W;
    const int j = seg - r * a.W;
    const int64_t seg_bytes = a.S * a.H * a.D * (int64_t)a.e;
    const uint8_t* src = a.base + (int64_t)r * a.stride + a.in_off + (int64_t)j * seg_bytes;
    uint8_t* dst = a.base + (int64_t)j * a.stride + a.stg_off + (int64_t)r * seg_bytes;
    copy_flat<V, 8>(src, dst, seg_bytes, (int64_t)blockIdx.x * kThreads + threadIdx.x,
                    (int64_t)gridDim.x * kThreads);
}

// Phase 2: staging_j[r][s][h][d] -> out_j[s][r*H + h][d]; rows (s, r) of H*D elements.
// (32-bit vector indices: the host checks S*W*H*D*e/V < 2^31 per destination.)
template <int V>
__global__ void __launch_bounds__(kThreads) two_phase_reorder_kernel(TwoPhaseArgs a) {
    using T = typename Vec<V>::T;
    const int j = blockIdx.y;
    const int64_t run = a.H * a.D * (int64_t)a.e;
    const int vpr = (int)(run / V);
    const int total = (int)(a.S * a.W * (int64_t)vpr);
    const int W = a.W;
    const int S = (int)a.S;
    const uint8_t* stg = a.base + (int64_t)j * a.stride + a.stg_off;
    T* out = reinterpret_cast<T*>(a.base + (int64_t)j * a.stride + a.out_off);
    constexpr int U = 8;
    const int nthr = (int)gridDim.x * kThreads;
    // destination order: row = s * W + r; source row (r, s) of staging_j
    auto src_of = [&](int idx) {
        const int row = idx / vpr;
        const int col = idx - row * vpr;
        const int s = row / W;
        const int r = row - s * W;
        return ((int64_t)r * S + s) * run + (int64_t)col * V;
    };
    int idx = (int)blockIdx.x * kThreads + (int)threadIdx.x;
    for (; idx + (U - 1) * nthr < total; idx += U * nthr) {
        T v[U];
        int64_t so[U];
#pragma unroll
        for (int u = 0; u < U; ++u) so[u] = src_of(idx + u * nthr);
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = *reinterpret_cast<const T*>(stg + so[u]);
#pragma unroll
        for (int u = 0; u < U; ++u) out[idx + u * nthr] = v[u];
    }
    for (; idx < total; idx += nthr) out[idx] = *reinterpret_cast<const T*>(stg + src_of(idx));
}

template <int V>
static hipError_t launch_two_phase_v(const TwoPhaseArgs& a, hipStream_t st) {
    const int64_t seg_bytes = a.S * a.H * a.D * (int64_t)a.e;
    const int64_t per_wg = (int64_t)kThreads * V * 8;
    int64_t gx = (seg_bytes + per_wg - 1) / per_wg;
    // enough workgroups in flight to fill 256 CUs; the grid-stride loop covers the rest
    const int64_t want = (2048 + (int64_t)a.W * a.W - 1) / ((int64_t)a.W * a.W);
    if (gx > want) gx = want;
    if (gx < 1) gx = 1;
    hipLaunchKernelGGL(two_phase_exchange_kernel<V>, dim3((unsigned)gx, a.W * a.W), dim3(kThreads),
                       0, st, a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    int64_t gx2 = 2048 / a.W;
    if (gx2 < 1) gx2 = 1;
    const int64_t need2 = (a.S * a.W * (a.H * a.D * (int64_t)a.e / V) + (int64_t)kThreads * 8 - 1) /
                          ((int64_t)kThreads * 8);
    if (gx2 > need2) gx2 = need2 > 0 ? need2 : 1;
    hipLaunchKernelGGL(two_phase_reorder_kernel<V>, dim3((unsigned)gx2, a.W), dim3(kThreads), 0, st,
                       a);
    return hipGetLastError();
}

hipError_t launch_two_phase(const TwoPhaseArgs& a, int V, hipStream_t st) {
    switch (V) {
        case 16: return launch_two_phase_v<16>(a, st);
        case 8: return launch_two_phase_v<8>(a, st);
        case 4: return launch_two_phase_v<4>(a, st);
        case 2: return launch_two_phase_v<2>(a, st);
        default: return launch_two_phase_v<1>(a, st);
    }
}

}  // namespace ra2a
