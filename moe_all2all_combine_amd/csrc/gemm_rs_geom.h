// Geometry of the GEMM + ReduceScatter overlap: the work queue of each stream
// group and the rows, columns and signals each task touches.  Shared by the
// gfx950 kernel and the host-side plan checker.
//
// (HyperParallel RFC, section 十 fused_matmul_reduce_scatter; "Triton-distributed
// Semantics", section "GEMM + ReduceScatter Overlapping".)  Rank r holds x1_r
// (m x K) and x2_r, passed transposed as x2_r^T (N x K); output =
// ReduceScatter(x1 @ x2): rank j receives out_j = rows [j*mj, (j+1)*mj) of
// sum_r x1_r @ x2_r, mj = m / W.  A task computes one kRsTileM x kRsTileN tile
// of rank r's partial for destination j.  The W - 1 tasks of the other ranks
// store their partials into j's receive area (slot r) and set the (tile, r)
// signal; the task of rank j itself -- the receiver's own partial, which never
// leaves its accumulators -- waits for those W - 1 signals, adds the partials in
// rank order (its own in its place) in fp32, stores the bf16 result and sets
// (tile, j).  A partial is the fp32 accumulator tile of x1_r @ x2_r, or
// optionally that product rounded to bf16 (nearest even), the type a
// framework's matmul returns.  Sources are visited in a rotation (the RFC's): at
// step s the producer for destination j is rank (j + 1 + s) mod W, so rank r
// works for rank (r - 1 - s) mod W, no destination is the target of every rank
// at once, and the receiver's own task comes last.
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
// Output tiles per queue block.
constexpr int kRsBlock = 32;

// A partial tile in the receive area: the 256 x 256 accumulators in the lanes'
// own order (fp32: [8 x 4 blocks][512 threads][4 values]; bf16: [8 x 2 block
// pairs][512 threads][2 x 4 values]), so that every store and load of a wave is
// 1 KiB contiguous and no LDS pass is needed on either side.  Rows and columns
// past the matrix hold zeros.
constexpr int64_t kRsPartElems = (int64_t)kRsTileM * kRsTileN;

struct GemmRsArgs {
    uint8_t* base;        // heap base (slice 0)
    int64_t stride;       // slice stride, bytes
    int64_t a_off;        // symmetric offset of x1 (x1_r in slice r), m x K bf16
    int64_t bt_off;       // symmetric offset of x2^T (x2_r^T in slice r), N x K bf16
    int64_t p_off;        // symmetric offset of the receive area: [W][ntiles] partial tiles in slice j
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
    int64_t ntasks_dest;  // queue tasks per destination: ntiles * W
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
    int j;        // destination rank
    int r;        // source rank; r == j: the receiver's own task, which adds the partials
    int tile;     // output tile index of out_j
};

// Queue of one destination: for each block b of kRsBlock tiles (the last may be
// shorter), its W x n_b tasks source-major in rotation order (step s = 0..W-1,
// source (j + 1 + s) mod W, then the block's tiles).  The receiver's task of a
// tile waits only for the other sources' tasks of that tile, all placed before
// it; no other task waits.  32-bit arithmetic: the host keeps positions below
// 2^31.
GRS_HD RsTask grs_task_of(const GemmRsArgs& a, int j, uint32_t pos) {
    const uint32_t W = (uint32_t)a.W, B = (uint32_t)kRsBlock;
    const uint32_t blk = pos / (W * B);
    const uint32_t n = (uint32_t)grs_block_tiles(a, (int)blk);
    const uint32_t q = pos - blk * W * B;
    const uint32_t s = q / n;
    RsTask t;
    t.j = j;
    t.r = (int)(((uint32_t)j + 1u + s) % W);
    t.tile = (int)(blk * B + (q - s * n));
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
// Partial tile of source r in j's receive area: byte offset of its slot (the
// receiver's own slot, r == j, is never written).
GRS_HD int64_t grs_part_offset(const GemmRsArgs& a, int r, int tile) {
    return ((int64_t)r * a.ntiles + tile) * kRsPartElems * (a.f32p ? 4 : 2);
}

}  // namespace ra2a
