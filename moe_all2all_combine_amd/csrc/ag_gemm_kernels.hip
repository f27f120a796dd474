// gfx950 kernel of the AllGather + GEMM overlap: one persistent launch whose
// workgroups take tasks from one work queue per XCD (queue.h):
//   * AllGather part: copy a few rows of shard w (slice w) into G (slice rank),
//     release, count the part; the tile's last part sets its signal to 1
//     (put_with_signal per tile, the HyperParallel RFC section 六 / 十);
//   * GEMM tile: wait until every tile covering its 256 rows is signalled,
//     then C[256 x 256] = G[rows, :] @ B[:, cols] on the matrix cores (bf16 in,
//     fp32 accumulation, bf16 out rounded to nearest even) -- "Triton-distributed
//     Semantics", sections "Producer-Consumer Model" and "AllGather + GEMM
//     Overlapping": the consumer waits only for its own tile.
//
// Shard w's tasks form stream group w mod NG, bound to one XCD (XCC_ID), so the
// rows a GEMM tile reads were written into the L2 it reads through; the part's
// release is then a drain plus a barrier (device.h).  With agent_sync the
// release writes the L2 back and the GEMM tile acquires device-wide instead.
#include <hip/hip_runtime.h>

#include "ag_gemm_geom.h"
#include "common.h"
#include "device.h"
#include "launch.h"
#include "queue.h"

namespace ra2a {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// LDS tile rows are padded from 64 to 72 bf16 (144 bytes): the 16-byte reads of
// 8 consecutive rows then start 4 banks apart and do not conflict.
constexpr int kLdsStride = kGemmBK + 8;
constexpr int kLdsOperand = kGemmBM * kLdsStride;  // bf16 elements of one operand stage

// float -> bf16, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint32_t bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

constexpr int kGemmThreads = 512;  // 8 waves: 2 (rows) x 4 (columns) of 128 x 64 each

// One pipeline stage's global loads per thread: 4 x 16 bytes of A (rows of G)
// and a 4 (k) x 8 (n) block of B.
struct StageRegs {
    u32x4 a[4];
    u32x4 b[4];
};

// Per-thread load cursor of a tile: thread t loads A rows t/8 + 64 i (i < 4),
// 16-byte chunk t % 8 of the stage's 64 k, and B rows k 4 (t % 16) + i (i < 4)
// at columns 8 (t / 16) .. +8.  Pointers advance by one stage per step.
// Out-of-range rows / columns / k read as zero.
struct StageCursor {
    const uint16_t* a;  // A row t/8, k of chunk t % 8, this stage
    const uint16_t* b;  // B row k 4 (t % 16), column 8 (t / 16), this stage
    int64_t ka, kb;     // k of the A chunk / of the first B row, this stage
    int arow;           // t / 8
    bool bn;            // the thread's 8 B columns are inside N
};

__device__ __forceinline__ void stage_load(StageRegs& r, const StageCursor& c, int rows_valid,
                                           int64_t K, int64_t N) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (c.arow + 64 * i < rows_valid && c.ka < K)
            v = *reinterpret_cast<const u32x4*>(c.a + (int64_t)(64 * i) * K);
        r.a[i] = v;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (c.kb + i < K && c.bn) v = *reinterpret_cast<const u32x4*>(c.b + (int64_t)i * N);
        r.b[i] = v;
    }
}

// Store a stage into LDS: A as loaded (row-major, k contiguous); B transposed
// in registers so that each column n holds consecutive k (the matrix cores take
// both operands k-contiguous): the 4 x 8 block becomes 8 columns of 4 k.
__device__ __forceinline__ void stage_store(const StageRegs& r, uint16_t* __restrict__ lds_a,
                                            uint16_t* __restrict__ lds_b) {
    const int t = (int)threadIdx.x;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = (t >> 3) + 64 * i;
        *reinterpret_cast<u32x4*>(lds_a + row * kLdsStride + 8 * (t & 7)) = r.a[i];
    }
    // r.b[kk] holds B[k = 4 (t%16) + kk][n = 8 (t/16) .. +8]: dword j packs columns 2j, 2j+1.
    // Column nn packs (k 0, k 1) in its first dword and (k 2, k 3) in its second.
    const int nbase = 8 * (t >> 4);
    const int kofs = 4 * (t & 15);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        u32x2 lo, hi;  // columns 2j and 2j + 1
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            lo[q] = __builtin_amdgcn_perm(r.b[2 * q + 1][j], r.b[2 * q][j], 0x05040100u);
            hi[q] = __builtin_amdgcn_perm(r.b[2 * q + 1][j], r.b[2 * q][j], 0x07060302u);
        }
        *reinterpret_cast<u32x2*>(lds_b + (nbase + 2 * j) * kLdsStride + kofs) = lo;
        *reinterpret_cast<u32x2*>(lds_b + (nbase + 2 * j + 1) * kLdsStride + kofs) = hi;
    }
}

// One stage of matrix-core work: wave (wm, wn) owns rows 128 wm .. +128 and
// columns 64 wn .. +64 of the tile as 4 x 2 blocks of 32 x 32; each k16 step
// reads 4 A and 2 B fragments (16 bytes per lane) and issues 8 MFMAs.
__device__ __forceinline__ void stage_mma(f32x16 (&acc)[4][2], const uint16_t* __restrict__ lds_a,
                                          const uint16_t* __restrict__ lds_b) {
    const int lane = (int)threadIdx.x & 63;
    const int wave = (int)threadIdx.x >> 6;
    const int wm = wave >> 2, wn = wave & 3;
    const int r = lane & 31;
    const int kh = 8 * (lane >> 5);
#pragma unroll
    for (int kk = 0; kk < kGemmBK / 16; ++kk) {
        bf16x8 fa[4], fb[2];
#pragma unroll
        for (int x = 0; x < 4; ++x)
            fa[x] = *reinterpret_cast<const bf16x8*>(lds_a + (128 * wm + 32 * x + r) * kLdsStride + 16 * kk + kh);
#pragma unroll
        for (int y = 0; y < 2; ++y)
            fb[y] = *reinterpret_cast<const bf16x8*>(lds_b + (64 * wn + 32 * y + r) * kLdsStride + 16 * kk + kh);
#pragma unroll
        for (int x = 0; x < 4; ++x)
#pragma unroll
            for (int y = 0; y < 2; ++y)
                acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[x], fb[y], acc[x][y], 0, 0, 0);
    }
}

// C[rows, cols] of one 256 x 256 output tile; rows of G start at g_rows.
__device__ __forceinline__ void gemm_tile(const AgGemmArgs& a, const uint16_t* __restrict__ g_rows,
                                          int rows_valid, int64_t n0, uint16_t* __restrict__ c_rows,
                                          uint16_t* __restrict__ lds) {
    // K and N opaque per tile: nothing derived from them is hoisted out of the
    // persistent task loop and kept alive across tiles.
    int64_t K = a.K, N = a.N;
    asm volatile("" : "+s"(K), "+s"(N));
    f32x16 acc[4][2];
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y) acc[x][y] = f32x16{};
    const int64_t nk = (K + kGemmBK - 1) / kGemmBK;
    const int t = (int)threadIdx.x;
    StageCursor cur;
    cur.arow = t >> 3;
    cur.ka = 8 * (t & 7);
    cur.a = g_rows + (int64_t)cur.arow * K + cur.ka;
    cur.kb = 4 * (t & 15);
    const int64_t n = n0 + 8 * (t >> 4);
    cur.bn = n < N;
    cur.b = a.b + cur.kb * N + n;
    StageRegs regs;
    stage_load(regs, cur, rows_valid, K, N);
    stage_store(regs, lds, lds + kLdsOperand);
    __syncthreads();
    for (int64_t s = 0; s < nk; ++s) {
        uint16_t* const cur_lds = lds + (s & 1) * 2 * kLdsOperand;
        uint16_t* const nxt_lds = lds + ((s + 1) & 1) * 2 * kLdsOperand;
        if (s + 1 < nk) {
            cur.a += kGemmBK;
            cur.ka += kGemmBK;
            cur.b += kGemmBK * N;
            cur.kb += kGemmBK;
            stage_load(regs, cur, rows_valid, K, N);
        }
        stage_mma(acc, cur_lds, cur_lds + kLdsOperand);
        if (s + 1 < nk) stage_store(regs, nxt_lds, nxt_lds + kLdsOperand);
        __syncthreads();
    }
    // epilogue: accumulator register e of block (x, y) holds row 8 (e/4) + 4 (lane/32) + e%4,
    // column lane % 32 of the block.  (The empty asm makes the output pointer opaque
    // here, so that the compiler does not hoist the epilogue's addresses above the
    // loop and keep them alive across it.)
    uint64_t cbase = reinterpret_cast<uint64_t>(c_rows);
    asm volatile("" : "+v"(cbase));
    c_rows = reinterpret_cast<uint16_t*>(cbase);
    const int lane = (int)threadIdx.x & 63;
    const int wave = (int)threadIdx.x >> 6;
    const int wm = wave >> 2, wn = wave & 3;
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y) {
            const int64_t col = n0 + 64 * wn + 32 * y + (lane & 31);  // < N checked below
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = 128 * wm + 32 * x + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                if (row < rows_valid && col < N)
                    c_rows[(int64_t)row * N + col] = (uint16_t)bf16_rne(acc[x][y][e]);
            }
        }
}

template <int SYNC>
__global__ void __launch_bounds__(kGemmThreads, 1) ag_gemm_kernel(AgGemmArgs a) {
    __shared__ uint16_t lds[4 * kLdsOperand];  // 2 stages x (A, B^T), 147456 bytes
    __shared__ int lds_flag;
    __shared__ int64_t lds_pos[2];
    constexpr bool kOwned = SYNC == kSyncXcd;
    uint8_t* const mine = a.base + (int64_t)a.rank * a.stride;
    uint64_t* const sig = reinterpret_cast<uint64_t*>(mine + a.sig_off);
    uint64_t* const qw = sig + agg_queue_slot(a) * kSigStrideU64;
    uint16_t* const G = reinterpret_cast<uint16_t*>(mine + a.g_off);
    const uint32_t xcc = xcc_id();
    const int home = SYNC == kSyncXcd ? (int)(xcc % (uint32_t)a.NG) : (int)(blockIdx.x % a.NG);
    const int64_t total = a.ntasks_shard * a.spg;
    QueueClaim qc;
    int k = 0;
    for (int gi = 0; gi < a.NG; ++gi) {
        const int g = (home + gi) % a.NG;
        if (threadIdx.x == 0) lds_pos[k & 1] = queue_first<kOwned>(qw, g, gi, xcc, qc);
        __syncthreads();
        int64_t pos = (int64_t)__builtin_amdgcn_readfirstlane((int)lds_pos[k & 1]);
        ++k;
        if (pos < 0) continue;
        while (true) {
            // the group's queue: spg shards of ntasks_shard each (the last group may
            // have fewer real shards; their tasks are skipped)
            if (pos >= total) {
                if (threadIdx.x == 0) queue_drained(qw, g, pos, total, qc);
                break;
            }
            uint64_t nxt = 0;
            if (threadIdx.x == 0) nxt = queue_next(qc);
            const AgTask t = agg_task_of(a, g, pos);
            if (t.w < a.W) {
                if (!t.gemm) {
                    // AllGather part: rows [row0, row0 + rows) of shard w -> G
                    const int64_t bytes = t.rows * a.K * 2;
                    const uint8_t* src = a.base + (int64_t)t.w * a.stride + a.a_off + t.row0 * a.K * 2;
                    uint8_t* dst = reinterpret_cast<uint8_t*>(G + ((int64_t)t.w * a.m_local + t.row0) * a.K);
                    copy_flat<16, 8>(src, dst, bytes, threadIdx.x, kGemmThreads);
                    group_release<SYNC>();
                    if (threadIdx.x == 0) {
                        const uint64_t done = __hip_atomic_fetch_add(sig + agg_count_slot(a, t.w, t.tile) * kSigStrideU64,
                                                                     1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        if (done + 1 == (uint64_t)agg_parts_of_tile(a, t.tile))
                            sig_update(sig + agg_sig_slot(a, t.w, t.tile) * kSigStrideU64, 1ull, kSigSet);
                    }
                } else {
                    int first, last;
                    agg_block_tiles(a, t.mb, &first, &last);
                    if (!group_wait_all<SYNC == kSyncAgent>(sig + agg_sig_slot(a, t.w, first) * kSigStrideU64,
                                                            kSigStrideU64 * 8, last - first, kCmpEq, 1ull,
                                                            a.timeout, a.err, &lds_flag))
                        return;
                    const int64_t row0 = (int64_t)t.w * a.m_local + (int64_t)t.mb * kGemmBM;
                    int64_t rv = a.m_local - (int64_t)t.mb * kGemmBM;
                    const int rows_valid = rv < kGemmBM ? (int)rv : kGemmBM;
                    gemm_tile(a, G + row0 * a.K, rows_valid, (int64_t)t.nb * kGemmBN, a.c + row0 * a.N, lds);
                }
            }
            if (threadIdx.x == 0) lds_pos[k & 1] = (int64_t)nxt;
            __syncthreads();
            pos = (int64_t)__builtin_amdgcn_readfirstlane((int)lds_pos[k & 1]);
            ++k;
        }
    }
}

hipError_t launch_ag_gemm(const AgGemmArgs& a, int grid, hipStream_t st) {
    void* args[] = {const_cast<AgGemmArgs*>(&a)};
    const void* fn = a.sync == kSyncXcd ? reinterpret_cast<const void*>(&ag_gemm_kernel<kSyncXcd>)
                                        : reinterpret_cast<const void*>(&ag_gemm_kernel<kSyncAgent>);
    return hipLaunchKernel(fn, dim3(grid), dim3(kGemmThreads), args, 0, st);
}

hipError_t ag_gemm_blocks_per_cu(int sync, int* n) {
    const void* fn = sync == kSyncXcd ? reinterpret_cast<const void*>(&ag_gemm_kernel<kSyncXcd>)
                                      : reinterpret_cast<const void*>(&ag_gemm_kernel<kSyncAgent>);
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(n, fn, kGemmThreads, 0);
}

}  // namespace ra2a
