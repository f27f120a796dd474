// Geometry of the GEMM + ReduceScatter overlap: the work queue of each stream
// group and the rows, columns and signals each task touches.  Shared by the
// gfx950 kernel and the host-side plan checker.
//
// (HyperParallel RFC, section 十 fused_matmul_reduce_scatter; "Triton-distributed
// Semantics", section "GEMM + ReduceScatter Overlapping".)  Rank r holds x1_r
// (m x K) and x2_r, passed transposed as x2_r^T (N x K); output =
// ReduceScatter(x1 @ x2): rank j receives out_j = rows [j*mj, (j+1)*mj) of
// sum_r x1_r @ x2_r, mj = m / W.  Producer tasks compute one kRsTileM x kRsTileN tile of
// rank r's partial for destination j and store it into j's receive area (slot
// r), then set the (tile, r) signal; the receiver's reduce task waits for the W
// partials of a tile, adds them in rank order in fp32 and stores the bf16 result.
// A partial is the fp32 accumulator tile of x1_r @ x2_r, or optionally that
// product rounded to bf16 (nearest even), the type a framework's matmul returns.  Sources are visited in the RFC's rotation: at step t the
// producer for destination j is rank (j - t) mod W, so rank r works for rank
// (r + t) mod W and no destination is the target of every rank at once.
#pragma once

#include <stdint.h>

#include "ag_gemm_geom.h"

#if defined(__HIPCC__)
#define GRS_HD __host__ __device__ __forceinline__
#else
#define GRS_HD inline
#endif

namespace ra2a {

// Output tiles are the GEMM tile of the matrix-core routine: kRsTileM rows of
// out_j by kRsTileN columns.
constexpr int kRsTileM = kGemmBM;
constexpr int kRsTileN = kGemmBN;
// Output tiles per queue block.  Measured at W = 8, m = 8192, K = 896, N = 4096
// (fp32 partials): while a reduce task waited for each partial load before
// issuing the next, blocks of 8 / 16 / 32 / 64 tiles took 1.105 / 1.017 / 0.991
// / 0.994 ms (a slow reduce among the GEMM tasks held compute up); with the loads
// of a reduce in flight together, 8 / 16 / 32 take 0.914 / 0.940 / 0.923-0.942 ms,
// the same within the run-to-run spread.
constexpr int kRsBlock = 32;

struct GemmRsArgs {
    uint8_t* base;        // heap base (slice 0)
    int64_t stride;       // slice stride, bytes
    int64_t a_off;        // symmetric offset of x1 (x1_r in slice r), m x K bf16
    int64_t bt_off;       // symmetric offset of x2^T (x2_r^T in slice r), N x K bf16
    int64_t p_off;        // symmetric offset of the receive area: [W][mj][N] bf16 (f32p: fp32) in slice j
    int64_t out_off;      // symmetric offset of out (out_j in slice j), mj x N bf16
    int64_t sig_off;      // symmetric offset of the signals ([tile][source] in slice j)
    uint32_t* err;
    uint64_t timeout;
    int32_t W;
    int64_t m, mj, K, N;
    int32_t ntm, ntn;     // output tiles of out_j along rows and columns
    int32_t ntiles;       // ntm * ntn
    int32_t nblocks;      // ceil(ntiles / kRsBlock)
    int32_t NG;           // stream groups (one per XCD)
    int32_t dpg;          // destinations per group: j = g, g + NG, ...
    int32_t sync;         // kSyncXcd | kSyncAgent
    int32_t f32p;         // 1: partials kept in fp32; 0: rounded to bf16 (a framework matmul's type)
    int64_t ntasks_dest;  // queue tasks per destination: ntiles * (W + 1)
};

// Output tile t of out_j: tiles are numbered in column groups of kRsBlock (for
// each group of kRsBlock column blocks, every row block), so the tiles of one
// queue block share row blocks of x1 and column blocks of x2.
GRS_HD void grs_tile(const GemmRsArgs& a, int t, int* mb, int* nb) {
    const int per_group = a.ntm * kRsBlock;
    const int ng = t / per_group;
    const int q = t - ng * per_group;
    const int width = a.ntn - ng * kRsBlock < kRsBlock ? a.ntn - ng * kRsBlock : kRsBlock;
    *mb = q / width;
    *nb = ng * kRsBlock + (q - *mb * width);
}

GRS_HD int grs_block_tiles(const GemmRsArgs& a, int blk) {
    const int t0 = blk * kRsBlock;
    return a.ntiles - t0 < kRsBlock ? a.ntiles - t0 : kRsBlock;
}

struct RsTask {
    bool reduce;
    int j;        // destination rank
    int r;        // source rank (GEMM tasks)
    int tile;     // output tile index of out_j
};

// Queue of one destination: for each block b of kRsBlock tiles, the W x n_b
// GEMM tasks of block b (source-major in rotation order: step s = 0..W-1,
// source (j - s) mod W, then the block's tiles), followed by the reduce tasks of
// block b - 1; the reduce tasks of the last block close the queue.  A reduce
// task waits only for GEMM tasks placed before it; GEMM tasks wait for nothing.
// Every block but the last holds kRsBlock tiles, so the segment of block b >= 1
// (its GEMM tasks, then block b - 1's reduce tasks) has (W + 1) kRsBlock tasks
// except the last one.  32-bit arithmetic: the host keeps positions below 2^31.
GRS_HD RsTask grs_task_of(const GemmRsArgs& a, int j, uint32_t pos) {
    const uint32_t W = (uint32_t)a.W, B = (uint32_t)kRsBlock;
    const uint32_t last = (uint32_t)a.nblocks - 1u;
    const uint32_t nl = (uint32_t)grs_block_tiles(a, (int)last);  // tiles of the last block
    RsTask t;
    t.j = j;
    t.r = 0;
    t.reduce = false;
    // GEMM task q of a block of n tiles: step s = q / n, tile q mod n
    auto gemm = [&](uint32_t blk, uint32_t q, uint32_t n) {
        const uint32_t s = q / n;
        t.r = (int)(((uint32_t)j + W - s % W) % W);
        t.tile = (int)(blk * B + (q - s * n));
    };
    if (last == 0u) {
        if (pos < W * nl) {
            gemm(0u, pos, nl);
        } else {
            t.reduce = true;
            t.tile = (int)(pos - W * nl);
        }
        return t;
    }
    if (pos < W * B) {
        gemm(0u, pos, B);
        return t;
    }
    uint32_t p = pos - W * B;
    const uint32_t segf = (W + 1u) * B;  // a full segment
    const uint32_t nfull = last - 1u;     // blocks 1 .. last - 1
    if (p < nfull * segf) {
        const uint32_t k = p / segf;
        const uint32_t q = p - k * segf;
        if (q < W * B) {
            gemm(k + 1u, q, B);
        } else {
            t.reduce = true;
            t.tile = (int)(k * B + (q - W * B));
        }
        return t;
    }
    p -= nfull * segf;
    if (p < W * nl) {  // GEMM tasks of the last block
        gemm(last, p, nl);
        return t;
    }
    p -= W * nl;
    t.reduce = true;  // reduce tasks of the last two blocks, in tile order
    t.tile = (int)((last - 1u) * B + p);
    return t;
}

// Task pos of group g: the group's destinations g, g + NG, ... one after another.
GRS_HD RsTask grs_group_task(const GemmRsArgs& a, int g, int64_t pos) {
    const uint32_t per = (uint32_t)a.ntasks_dest;
    const uint32_t di = (uint32_t)pos / per;
    return grs_task_of(a, g + (int)di * a.NG, (uint32_t)pos - di * per);
}

// Signal slots (in slice j): [tile][source], then (slice 0) the queue words.
GRS_HD int64_t grs_sig_slot(const GemmRsArgs& a, int tile, int r) { return (int64_t)tile * a.W + r; }
GRS_HD int64_t grs_queue_slot(const GemmRsArgs& a) { return (int64_t)a.ntiles * a.W; }

}  // namespace ra2a
