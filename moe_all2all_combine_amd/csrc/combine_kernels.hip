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

namespace ra2a {

// ---------------------------------------------------------------------------
// Signal reset: slot i of every slice r (8 bytes at 128-byte spacing) := 0.
// ("Host Side Modifications": every signal is zeroed before each launch.)
__global__ void __launch_bounds__(kThreads) signal_reset_kernel(uint8_t* base, int64_t stride,
                                                                int W, int64_t sig_off,
                                                                int64_t nslots) {
    const int64_t total = (int64_t)W * nslots;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = i / nslots;
        const int64_t k = i - r * nslots;
        uint64_t* p = reinterpret_cast<uint64_t*>(base + r * stride + sig_off) + k * kSigStrideU64;
        *p = 0ull;
    }
}

hipError_t launch_signal_reset(uint8_t* base, int64_t stride, int W, int64_t sig_off,
                               int64_t nslots, hipStream_t st) {
    const int64_t total = (int64_t)W * nslots;
    if (total <= 0) return hipSuccess;
    int64_t blocks = (total + kThreads - 1) / kThreads;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(signal_reset_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, st, base,
                       stride, W, sig_off, nslots);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Copies vectors [lo, hi) of a row plan (combine_geom.h).  Full rounds keep U
// vectors per thread in flight (all loads before any store, no bounds checks
// so the values stay in registers); the remainder goes one vector at a time.
// NTL / NTS: non-temporal loads / stores (data touched once: the input and the
// output), so that they do not displace the staging ring from the L2.
template <int V, int U, bool NTL, bool NTS>
__device__ __forceinline__ void copy_plan(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                          const RowPlan& p, int lo, int hi) {
    using T = typename Vec<V>::T;
    const int vpr = p.run / V;
    const int BC = p.B * p.C;
    for (int base = lo + (int)threadIdx.x; base < hi; base += U * kThreads) {
        // predicated round: every load of the round is issued before any store
        T v[U];
        int64_t doff[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int idx = base + u * kThreads;
            int64_t so = 0;
            doff[u] = -1;
            if (idx < hi) plan_offsets(p, V, vpr, BC, idx, &so, &doff[u]);
            const T* sp = reinterpret_cast<const T*>(src + so);
            if (idx < hi) v[u] = NTL ? load_nt(sp) : *sp;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (doff[u] >= 0) {
                T* dp = reinterpret_cast<T*>(dst + doff[u]);
                if (NTS)
                    store_nt(v[u], dp);
                else
                    *dp = v[u];
            }
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
    const int vpr = p.run / V;
    const int BC = p.B * p.C;
    for (int base = lo + (int)threadIdx.x; base < hi; base += U * kThreads) {
        T v[U];
        int64_t doff[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int idx = base + u * kThreads;
            int64_t so = 0;
            doff[u] = -1;
            if (idx < hi) plan_offsets(p, V, vpr, BC, idx, &so, &doff[u]);
            if (idx < hi) v[u] = BufLoad<V, POLICY>::go(src, src_off + (uint32_t)so);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (doff[u] >= 0) {
                T* dp = reinterpret_cast<T*>(dst + doff[u]);
                if (NTS)
                    store_nt(v[u], dp);
                else
                    *dp = v[u];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// The signal-pipelined persistent combine.
//
// Work is organised in tile streams: stream (j, hb, db) is the sequence of
// S-blocks b = 0 .. nbs-1 of destination j, head block hb, d block db.  The
// streams are cut into NG contiguous groups; group g is served by the
// workgroups w with w mod NG == g.  With NG equal to the number of XCDs that
// is exactly the set of workgroups the dispatcher places on XCD g (checked at
// run time through the XCC_ID hardware register), so a stream's producers,
// consumers, staging lines and signals all live in one XCD and its L2, and
// they synchronise with the XCD-local sequences of device.h instead of device-
// wide L2 write-backs and invalidations (SYNC == kSyncXcd).  SYNC == kSyncAgent
// uses device-wide release/acquire instead and does not depend on placement.
//
// Inside a group, tiles (stream, S-block) are ordered by stream batch (KB
// streams whose staging is live together), S-block, stream; the workgroups
// alternate roles with period q: the first p of each period produce, the rest
// consume.
//
// Producer: pieces (tile, source r) of its group in order, `pbatch`
// consecutive pieces per turn.  Per piece: wait for the ring slot b mod R of
// its stream to be handed back by the consumers of S-block b - R (credit
// count), copy in_r -> staging_j.  Per turn: release, then wave 0 signals
// each piece (SET 1 on the piece's slot, or ADD 1 on the tile's slot).  Pieces
// already copied in a turn are signalled before any hand-back wait of that
// turn.
//
// Consumer: units of its group in order (ADD: a tile with all W sources; SET:
// one piece), each split into `csplit` parts taken by different workgroups.
// Per part: wait until the signal reaches W (ADD) or 1 (SET), acquire, copy
// staging_j -> out_j, release, add 1 to the slot's credit count.
//
// Deadlock freedom: the launch is cooperative (every workgroup resident), each
// workgroup walks its work in increasing tile order, a producer of tile
// (k, b) waits only on consumers of the earlier tile (k, b - R) and a consumer
// only on producers of its own tile; so the earliest blocked wait always has a
// running workgroup able to satisfy it.  Every wait is also bounded in time.
template <int V, int SYNC>
__global__ void __launch_bounds__(kThreads) rev_a2a_pipelined_kernel(PipeArgs a) {
    __shared__ int lds_flag;
    const Role role = role_of(a, blockIdx.x);
    const int g = role.g;
    const bool add = a.protocol == kSigAdd;
    uint8_t* const base = a.base;
    if (SYNC == kSyncXcd && threadIdx.x == 0 && (int)xcc_id() != (int)(blockIdx.x % a.NG))
        __hip_atomic_fetch_or(a.err, kErrPlacement, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

    if (role.producer) {
        const int64_t npieces = group_pieces(a, g);
        // Publish pieces [lo, hi) of this workgroup: release, then wave 0 signals each.
        auto flush = [&](int64_t lo, int64_t hi) {
            group_release<SYNC>();
            if (threadIdx.x < 64) {
                for (int64_t pc = lo + threadIdx.x; pc < hi; pc += 64) {
                    const Piece p = piece_of(a, g, pc);
                    sig_update(reinterpret_cast<uint64_t*>(base + p.sig), 1ull,
                                           add ? kSigAdd : kSigSet);
                }
            }
        };
        for (int64_t first = (int64_t)role.index * a.pbatch; first < npieces;
             first += (int64_t)a.nprod * a.pbatch) {
            const int64_t last = min(first + (int64_t)a.pbatch, npieces);
            int64_t pend = first;  // first piece of this turn not yet signalled
            for (int64_t pc = first; pc < last; ++pc) {
                const Piece p = piece_of(a, g, pc);
                if (p.b >= a.R) {
                    // Signal what this turn already copied before blocking on a hand-back:
                    // that hand-back may depend on those very pieces.
                    if (pc > pend) {
                        flush(pend, pc);
                        pend = pc;
                    }
                    if (!group_wait<false>(reinterpret_cast<const uint64_t*>(base + p.credit),
                                           kCmpGe, p.credit_need, a.timeout, a.err, &lds_flag))
                        return;
                }
                if (p.r == a.straggler && a.delay) {
                    if (threadIdx.x == 0) {
                        const uint64_t id = ((uint64_t)p.b * (uint64_t)a.nstreams + p.sid) * a.W + p.r;
                        const uint64_t n =
                            a.delay + splitmix64(a.seed, id) % ((uint64_t)a.delay + 1ull);
                        for (uint64_t i = 0; i < n; ++i) __builtin_amdgcn_s_sleep(1);
                    }
                    __syncthreads();
                }
                copy_plan<V, 8, true, false>(base + p.src, base + p.dst, p.pl, 0,
                                             plan_vectors(p.pl, V));
            }
            flush(pend, last);
        }
    } else {
        const int64_t nitems = group_items(a, g);
        for (int64_t it = role.index; it < nitems; it += a.ncons) {
            const Item q = item_of(a, g, it, V);
            // XCD-local: staging is read with device-scope (L1-bypassing) loads from
            // the L2 this XCD's producers wrote it into, so no invalidation is needed.
            // Device-wide: the acquire drops stale L1 and L2 lines first.
            if (!group_wait<SYNC == kSyncAgent>(reinterpret_cast<const uint64_t*>(base + q.sig),
                                                kCmpEq, q.sig_want, a.timeout, a.err, &lds_flag))
                return;
            if (SYNC == kSyncXcd) {
                const int64_t stg = (int64_t)q.j * a.stride + a.stg_off;
                copy_plan_buf<V, 8, kPolicySc1, true>(make_rsrc(base + stg, (uint32_t)a.ring_bytes),
                                                      (uint32_t)(q.src - stg), base + q.dst, q.pl,
                                                      q.lo, q.hi);
            } else {
                copy_plan<V, 8, false, true>(base + q.src, base + q.dst, q.pl, q.lo, q.hi);
            }
            group_release<SYNC>();
            if (threadIdx.x == 0) {
                sig_update(reinterpret_cast<uint64_t*>(base + q.credit), 1ull,
                                       kSigAdd);
                if (a.stamps)
                    __hip_atomic_fetch_max(a.stamps + (int64_t)q.j * a.units_per_dest + q.unit_index,
                                           rtc_now(), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
}

template <int V, int SYNC>
static const void* pipelined_fn() {
    return reinterpret_cast<const void*>(&rev_a2a_pipelined_kernel<V, SYNC>);
}

template <int SYNC>
static const void* pipelined_fn_v(int V) {
    switch (V) {
        case 16: return pipelined_fn<16, SYNC>();
        case 8: return pipelined_fn<8, SYNC>();
        case 4: return pipelined_fn<4, SYNC>();
        case 2: return pipelined_fn<2, SYNC>();
        default: return pipelined_fn<1, SYNC>();
    }
}

static const void* pipelined_kernel(int V, int sync) {
    return sync == kSyncXcd ? pipelined_fn_v<kSyncXcd>(V) : pipelined_fn_v<kSyncAgent>(V);
}

hipError_t launch_pipelined(const PipeArgs& a, int V, int grid, hipStream_t st) {
    void* args[] = {const_cast<PipeArgs*>(&a)};
    return hipLaunchCooperativeKernel(pipelined_kernel(V, a.sync), dim3(grid), dim3(kThreads), args,
                                      0, st);
}

hipError_t pipelined_blocks_per_cu(int V, int sync, int* n) {
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(n, pipelined_kernel(V, sync), kThreads, 0);
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
