// gfx950 kernels of the Reverse All2All combine:
//   * signal_reset  -- zero signal slots in every slice before a launch;
//   * rev_a2a_pipelined -- persistent, role-split, tile-signalled combine;
//   * two_phase_exchange / two_phase_reorder -- the exchange-then-reorder variant.
//
// Combine ("Reverse All2All (EP MoE Distributed Kernel)", section "Reverse
// All2All Operator Semantics"): out_j[s, r*H + h, d] = in_r[j*S + s, h, d].
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
        if (threadIdx.x == 0) {
            const uint64_t id = ((uint64_t)p.b * (uint64_t)a.nstreams + p.sid) * a.W + p.r;
            const uint64_t n = a.delay + splitmix64(a.seed, id) % ((uint64_t)a.delay + 1ull);
            for (uint64_t i = 0; i < n; ++i) __builtin_amdgcn_s_sleep(1);
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

// Before a workgroup's first signal: every reset flag carries this launch's tag
// (lane k of wave 0 polls flag k), then wave 0 -- the one that signals and
// stamps -- acquires.  False, uniformly, if a bounded wait gave up.
__device__ __forceinline__ bool reset_published(const PipeArgs& a) {
    bool ok = true;
    if ((int)threadIdx.x < a.reset_nz)
        ok = spin_until(reinterpret_cast<const uint64_t*>(a.base + a.flag_off) +
                            (int64_t)threadIdx.x * kSigStrideU64,
                        kCmpEq, a.reset_tag, a.timeout, a.err);
    if (threadIdx.x < 64) fence_acquire_agent();
    return __syncthreads_and(ok ? 1 : 0) != 0;
}

// Direct mode.  Producers store straight into out_j, so no consumer has data to
// move: a tile is complete when its signal reaches W (ADD) or each of its W
// slots reads 1 (SET), and the optional completion stamp of a tile is the
// latest of its producers' stamps (an atomic max each).  The only wait is for
// the in-launch reset's flags (above), so a static schedule (workgroup k takes
// pieces k, k + piece_grid, ... of the direct_piece order) needs no queue.  The
// reset runs on reset_nz workgroups launched after the piece_grid ones, and the
// host launches it only when the occupancy leaves room for them beside the
// persistent workgroups: they run whatever those do and wait on nothing, so
// the wait always ends.  Every atomic is issued without a return value, so no
// drain waits for a round trip.  A piece's geometry is 32-bit scalar arithmetic: the inline 64-bit
// division sequences it replaced delayed every piece's first load measurably.
// (Measured too: issuing the next piece's loads before this piece's release is
// slower here, not faster.)
template <int V, int SYNC>
__device__ __forceinline__ void direct_path(const PipeArgs& a, int* lds_flag) {
    const int pg = a.piece_grid;
    if ((int)blockIdx.x >= pg) {  // a zeroing workgroup of the in-launch reset
        reset_share(a, (int)blockIdx.x - pg);
        return;
    }
    bool published = a.reset_tag == 0ull;
    const int64_t total = total_pieces(a);
    for (int64_t gp = blockIdx.x; gp < total; gp += pg) {
        const Piece p = direct_piece(a, gp);
        if (!piece_wait(a, p, lds_flag)) return;
        // final place: stream the stores past the L2
        copy_plan<V, 8, true, true>(a.base + p.src, a.base + p.dst, p.pl, 0, plan_vectors(p.pl, V));
        group_release<SYNC>();
        if (!published) {
            if (!reset_published(a)) return;
            published = true;
        }
        piece_signal(a, p.sig, p.sig_step, p.nsig);
        if (a.stamps && threadIdx.x < 64) {
            const uint64_t now = rtc_now();
            const int64_t step = slot_step(a);
            for (int k = threadIdx.x; k < p.nsig; k += 64)
                __hip_atomic_fetch_max(a.stamps + (int64_t)p.j * a.units_per_dest + p.unit_index + k * step,
                                       now, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

template <int V, int SYNC, bool DIRECT>
__global__ void __launch_bounds__(kThreads) rev_a2a_pipelined_kernel(PipeArgs a) {
    __shared__ int lds_flag;
    __shared__ int64_t lds_pos[2];
    if (DIRECT) {
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
