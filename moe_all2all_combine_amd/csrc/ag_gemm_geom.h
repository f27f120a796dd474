// Geometry of the AllGather + GEMM overlap: the work queue of each stream group
// (AllGather parts and GEMM output tiles) and the rows / signals each task
// touches.  Shared by the gfx950 kernel and the host-side plan checker.
//
// ("Triton-distributed Semantics", section "AllGather + GEMM Overlapping"; the
// HyperParallel RFC, section 十 fused_all_gather_matmul.)  W row shards A_w
// (m_local x K, bf16, shard w in heap slice w) are gathered into G (W*m_local x
// K) in the gathering rank's slice, shard w at rows [w*m_local, (w+1)*m_local);
// C = G @ B with B (K x N) and C (W*m_local x N), bf16 in and out, fp32
// accumulation.  Each tile of `tile_rows` rows of a shard is put with a signal
// (SET 1 once all its parts are in G); a GEMM tile waits only for the tiles
// covering its own rows.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define AGG_HD __host__ __device__ __forceinline__
#else
#define AGG_HD inline
#endif

namespace ra2a {

constexpr int kGemmBM = 256;  // GEMM output tile rows
constexpr int kGemmBN = 256;  // GEMM output tile columns

struct AgGemmArgs {
    uint8_t* base;        // heap base (slice 0)
    int64_t stride;       // slice stride, bytes
    int64_t a_off;        // symmetric offset of the shards (shard w in slice w)
    int64_t g_off;        // symmetric offset of G (used in slice `rank`)
    int64_t sig_off;      // symmetric offset of the signals (used in slice `rank`)
    const uint16_t* bt;   // B^T, N x K row-major bf16 (B transposed)
    uint16_t* c;          // C, (W*m_local) x N row-major bf16
    uint32_t* err;
    uint64_t timeout;
    int32_t W, rank;
    int64_t m_local, K, N;
    int32_t tile_rows;    // rows per signalled AllGather tile
    int32_t ntiles;       // AllGather tiles per shard
    int32_t rpp;          // rows per AllGather part (a part never straddles tiles)
    int32_t np;           // parts of a full tile
    int32_t np_last;      // parts of the last tile
    int32_t nmb;          // GEMM row blocks per shard
    int32_t ncol;         // GEMM column blocks
    int32_t NG;           // stream groups (one per XCD)
    int32_t spg;          // shards per group: shards g, g + NG, g + 2 NG, ...
    int32_t sync;         // kSyncXcd | kSyncAgent
    int64_t ntasks_shard; // tasks per shard
};

// Parts of the tiles [0, t).
AGG_HD int64_t agg_parts_before(const AgGemmArgs& a, int t) {
    if (t <= 0) return 0;
    if (t < a.ntiles) return (int64_t)t * a.np;
    return (int64_t)(a.ntiles - 1) * a.np + a.np_last;
}

// GEMM tiles are queued in groups of kColGroup column blocks: for each group,
// every row block of the shard, then every column block of the group.  The
// tiles a group keeps in flight on one XCD (its 32 compute units) then share
// row blocks of G and column blocks of B in the XCD's L2.
constexpr int kColGroup = 8;

AGG_HD int64_t agg_tasks_per_shard(const AgGemmArgs& a) {
    return (int64_t)a.nmb * a.ncol + agg_parts_before(a, a.ntiles);
}

struct AgTask {
    bool gemm;
    int w;        // shard
    // AllGather part
    int tile, part;
    int64_t row0, rows;   // rows of the shard
    // GEMM tile
    int mb, nb;
};

// Task at position pos of group g's queue.  A shard's queue holds all its
// AllGather parts (tile by tile), then its GEMM tiles in column-group order.
// Every GEMM tile follows all parts it waits for: every wait points backwards.
// (The parts are short copies; the GEMM tiles wait only for their own rows.)
AGG_HD AgTask agg_task_of(const AgGemmArgs& a, int g, int64_t pos) {
    AgTask t;
    const int64_t si = pos / a.ntasks_shard;
    const int64_t r = pos - si * a.ntasks_shard;
    t.w = g + (int)si * a.NG;
    const int64_t nparts = agg_parts_before(a, a.ntiles);
    if (r >= nparts) {
        const int64_t q = r - nparts;
        const int64_t per_group = (int64_t)a.nmb * kColGroup;
        const int ngroups = (a.ncol + kColGroup - 1) / kColGroup;
        int ng = (int)(q / per_group);
        if (ng > ngroups - 1) ng = ngroups - 1;
        const int64_t q1 = q - (int64_t)ng * per_group;
        const int width = a.ncol - ng * kColGroup < kColGroup ? a.ncol - ng * kColGroup : kColGroup;
        t.gemm = true;
        t.mb = (int)(q1 / width);
        t.nb = ng * kColGroup + (int)(q1 - (int64_t)t.mb * width);
        t.tile = t.part = 0;
        t.row0 = t.rows = 0;
        return t;
    }
    const int64_t part = r;
    t.gemm = false;
    t.mb = t.nb = 0;
    const int64_t full = (int64_t)(a.ntiles - 1) * a.np;
    if (part < full) {
        t.tile = (int)(part / a.np);
        t.part = (int)(part - (int64_t)t.tile * a.np);
    } else {
        t.tile = a.ntiles - 1;
        t.part = (int)(part - full);
    }
    const int64_t tile_end_row = (int64_t)(t.tile + 1) * a.tile_rows < a.m_local
                                     ? (int64_t)(t.tile + 1) * a.tile_rows
                                     : a.m_local;
    t.row0 = (int64_t)t.tile * a.tile_rows + (int64_t)t.part * a.rpp;
    const int64_t end = t.row0 + a.rpp < tile_end_row ? t.row0 + a.rpp : tile_end_row;
    t.rows = end - t.row0;
    return t;
}

// Tiles a GEMM row block waits for: [first, last).
AGG_HD void agg_block_tiles(const AgGemmArgs& a, int mb, int* first, int* last) {
    const int64_t r0 = (int64_t)mb * kGemmBM;
    int64_t r1 = r0 + kGemmBM;
    if (r1 > a.m_local) r1 = a.m_local;
    *first = (int)(r0 / a.tile_rows);
    *last = (int)((r1 + a.tile_rows - 1) / a.tile_rows);
}

// Signal slots (in the gathering rank's slice): [0, W*ntiles) tile signals
// (SET 1 when complete), [W*ntiles, 2*W*ntiles) part counters, then the queue
// words of the work queues.
AGG_HD int64_t agg_sig_slot(const AgGemmArgs& a, int w, int tile) { return (int64_t)w * a.ntiles + tile; }
AGG_HD int64_t agg_count_slot(const AgGemmArgs& a, int w, int tile) {
    return (int64_t)a.W * a.ntiles + (int64_t)w * a.ntiles + tile;
}
AGG_HD int64_t agg_queue_slot(const AgGemmArgs& a) { return 2 * (int64_t)a.W * a.ntiles; }

AGG_HD int agg_parts_of_tile(const AgGemmArgs& a, int tile) {
    return tile < a.ntiles - 1 ? a.np : a.np_last;
}

}  // namespace ra2a
