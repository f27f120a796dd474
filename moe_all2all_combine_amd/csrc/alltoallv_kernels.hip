// gfx950 kernel of the variable-size AllToAll (push): one persistent launch
// walking the work queue of alltoallv_geom.h (HyperParallel RFC, section 十,
// "AllToAll (Push mode)": metadata first, then every rank pushes its segments,
// and each destination's signal accumulates to the world size).
//
// Counts stay on the device: no host round trip between the metadata exchange
// and the data.  Every workgroup reads the W x W send counts once (inputs, not
// written during the launch), drops the counts of any sender whose counts are
// unusable, and builds the chunk table (exclusive prefix of chunks over the
// (sender, rotation step) pairs) in LDS, so that it can decode any queue
// position.  Positions are claimed in order from one atomic counter; a task
// waits only for tasks at earlier positions, so the earliest unfinished task
// can always proceed, whatever the number of resident workgroups.
//
// Memory ordering.  The metadata words (receive counts, offsets, chunk
// counters, arrival signals) are device-scope read-modify-write atomics and
// device-scope atomic loads, coherent across XCDs on their own; a writer drains
// (s_waitcnt vmcnt(0)) before the signal that publishes them.  The data rows
// are streamed with non-temporal loads and stores, drained before the chunk
// counter moves; no workgroup of the launch reads them back.
#include <hip/hip_runtime.h>

#include "alltoallv_geom.h"
#include "common.h"
#include "device.h"
#include "launch.h"

namespace ra2a {

namespace {

__device__ __forceinline__ uint64_t* a2v_sig(const A2vArgs& a, int slice, int64_t slot) {
    return reinterpret_cast<uint64_t*>(a.base + (int64_t)slice * a.stride + a.sig_off) + slot * kSigStrideU64;
}

__device__ __forceinline__ uint64_t* a2v_recv_count(const A2vArgs& a, int j, int r) {
    return reinterpret_cast<uint64_t*>(a.base + (int64_t)j * a.stride + a.rc_off) + r;
}

// Lane 0 waits until *p satisfies (op, v) and hands the value it saw to the
// whole workgroup.  False, uniformly, if the bounded wait gave up.
__device__ __forceinline__ bool wg_wait_value(const A2vArgs& a, const uint64_t* p, int op, uint64_t v,
                                              uint64_t* seen, uint64_t* lds_val, int* lds_flag) {
    if (threadIdx.x == 0) {
        const bool ok = spin_until(p, op, v, a.timeout, a.err);
        *lds_val = ok ? sig_load(p) : 0ull;
        *lds_flag = ok ? 1 : 0;
    }
    __syncthreads();
    const bool ok = *lds_flag != 0;
    *seen = *lds_val;
    __syncthreads();
    return ok;
}

// Inclusive prefix sum of x over the 64 lanes of a wave.
__device__ __forceinline__ int64_t wave_inclusive_scan(int64_t x) {
    const int lane = (int)threadIdx.x & 63;
    for (int d = 1; d < 64; d <<= 1) {
        const int64_t up = __shfl_up(x, d, 64);
        if (lane >= d) x += up;
    }
    return x;
}

}  // namespace

template <int V>
__global__ void __launch_bounds__(kThreads) alltoallv_kernel(A2vArgs a) {
    __shared__ int64_t cnt[kA2vMaxW * kA2vMaxW];        // usable send counts, [r][j]
    __shared__ int64_t first[kA2vMaxW * kA2vMaxW + 1];  // chunk table over (r, t) pairs
    __shared__ int rank_ok[kA2vMaxW];
    __shared__ int64_t lds_pos;
    __shared__ uint64_t lds_val;
    __shared__ int lds_flag;
    const int W = a.W;
    const int n = W * W;
    const int tid = (int)threadIdx.x;

    // ---- the counts and the chunk table ----
    for (int i = tid; i < n; i += kThreads) {
        const int r = i / W, j = i - (i / W) * W;
        cnt[i] = *reinterpret_cast<const int64_t*>(a.base + (int64_t)r * a.stride + a.cnt_off + j * 8);
    }
    __syncthreads();
    if (tid < W) rank_ok[tid] = a2v_rank_ok(W, a.in_rows, cnt + tid * W) ? 1 : 0;
    __syncthreads();
    for (int i = tid; i < n; i += kThreads)
        if (!rank_ok[i / W]) cnt[i] = 0;
    __syncthreads();
    if (tid < 64) {
        // wave 0: lane L owns pairs [L*per, (L+1)*per); exclusive scan across lanes
        const int per = (n + 63) / 64;
        int64_t local = 0;
        for (int k = 0; k < per; ++k) {
            const int p = tid * per + k;
            if (p < n) {
                const int r = p / W;
                local += a2v_chunks(cnt[r * W + a2v_dest(W, r, p - r * W)], a.row_bytes, a.chunk);
            }
        }
        const int64_t incl = wave_inclusive_scan(local);
        int64_t run = incl - local;
        for (int k = 0; k < per; ++k) {
            const int p = tid * per + k;
            if (p < n) {
                first[p] = run;
                const int r = p / W;
                run += a2v_chunks(cnt[r * W + a2v_dest(W, r, p - r * W)], a.row_bytes, a.chunk);
            }
        }
        if (tid == 63) first[n] = incl;
    }
    __syncthreads();

    // ---- the queue ----
    uint64_t* const qc = a2v_sig(a, 0, a2v_queue_slot(W));
    const int64_t total = a2v_total(W, first);
    if (tid == 0) lds_pos = (int64_t)__hip_atomic_fetch_add(qc, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    int64_t pos = lds_pos;
    __syncthreads();
    while (pos < total) {
        uint64_t nxt = 0;
        if (tid == 0) nxt = __hip_atomic_fetch_add(qc, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const A2vTask t = a2v_task(W, first, pos);
        if (t.kind == 0) {
            // sender r: its usable count for each destination into recv_counts_j[r],
            // then (once they are in) one ADD on each destination's count signal
            if (tid < W) sig_update(a2v_recv_count(a, tid, t.r), (uint64_t)cnt[t.r * W + tid], kSigSet);
            if (tid == 0 && !rank_ok[t.r])
                __hip_atomic_fetch_or(a.err, kErrCounts, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            group_release<kSyncXcd>();
            if (tid < W) sig_update(a2v_sig(a, tid, a2v_count_slot()), 1ull, kSigAdd);
        } else if (t.kind == 1) {
            // destination j: once every sender's count is in, hand each sender r the
            // first row of its rows in out_j (+1, so that 0 means "not yet")
            uint64_t seen;
            if (!wg_wait_value(a, a2v_sig(a, t.j, a2v_count_slot()), kCmpEq, (uint64_t)W, &seen, &lds_val,
                               &lds_flag))
                return;
            if (tid < 64) {  // lane r: sender r's count, then its exclusive prefix
                const int64_t c = tid < W ? (int64_t)sig_load(a2v_recv_count(a, t.j, tid)) : 0;
                const int64_t before = wave_inclusive_scan(c) - c;
                if (tid < W) sig_update(a2v_sig(a, tid, a2v_offset_slot(t.j)), (uint64_t)before + 1ull, kSigSet);
            }
        } else if (t.kind == 2) {
            // chunk c of sender r's segment for j
            uint64_t seen;
            if (!wg_wait_value(a, a2v_sig(a, t.r, a2v_offset_slot(t.j)), kCmpNe, 0ull, &seen, &lds_val,
                               &lds_flag))
                return;
            const int64_t rows = cnt[t.r * W + t.j];
            const int64_t dst_row = (int64_t)seen - 1;
            // (written so that a garbage offset -- signals not reset -- can neither
            // pass with a negative row nor overflow the sum)
            if (dst_row >= 0 && rows <= a.out_rows && dst_row <= a.out_rows - rows) {
                int64_t lo, hi;
                a2v_chunk_range(rows, a.row_bytes, a.chunk, t.c, &lo, &hi);
                const int64_t src_row = a2v_send_offset(W, cnt, t.r, t.j);
                const uint8_t* src = a.base + (int64_t)t.r * a.stride + a.in_off + src_row * a.row_bytes + lo;
                uint8_t* dst = a.base + (int64_t)t.j * a.stride + a.out_off + dst_row * a.row_bytes + lo;
                copy_flat<V, 8, true>(src, dst, hi - lo, tid, kThreads);
            } else if (tid == 0) {
                __hip_atomic_fetch_or(a.err, kErrOverflow, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            group_release<kSyncXcd>();
            if (tid == 0) {
                const uint64_t done = __hip_atomic_fetch_add(a2v_sig(a, t.j, a2v_chunk_slot(W, t.r)), 1ull,
                                                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (done + 1ull == (uint64_t)a2v_chunks(rows, a.row_bytes, a.chunk))
                    sig_update(a2v_sig(a, t.j, a2v_arrival_slot(W)), 1ull, kSigAdd);
            }
        } else if (t.kind == 3) {
            // destination j: every sender's segment has arrived; publish the total
            uint64_t seen;
            if (!wg_wait_value(a, a2v_sig(a, t.j, a2v_arrival_slot(W)), kCmpEq, (uint64_t)W, &seen, &lds_val,
                               &lds_flag))
                return;
            if (tid < 64) {
                const int64_t c = tid < W ? (int64_t)sig_load(a2v_recv_count(a, t.j, tid)) : 0;
                const int64_t sum = wave_inclusive_scan(c);
                if (tid == 63) sig_update(a2v_recv_count(a, t.j, W), (uint64_t)sum, kSigSet);
            }
        }
        if (tid == 0) lds_pos = (int64_t)nxt;
        __syncthreads();
        pos = lds_pos;
        __syncthreads();
    }
}

static const void* alltoallv_fn(int V) {
    switch (V) {
        case 16: return reinterpret_cast<const void*>(&alltoallv_kernel<16>);
        case 4: return reinterpret_cast<const void*>(&alltoallv_kernel<4>);
        default: return reinterpret_cast<const void*>(&alltoallv_kernel<1>);
    }
}

hipError_t launch_alltoallv(const A2vArgs& a, int V, int grid, hipStream_t st) {
    void* args[] = {const_cast<A2vArgs*>(&a)};
    return hipLaunchKernel(alltoallv_fn(V), dim3(grid), dim3(kThreads), args, 0, st);
}

hipError_t alltoallv_blocks_per_cu(int V, int* n) {
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(n, alltoallv_fn(V), kThreads, 0);
}

}  // namespace ra2a
