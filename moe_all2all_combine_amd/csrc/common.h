// Constants and launch-argument structs shared by the host code and the kernels.
#pragma once

#include <stdint.h>

namespace ra2a {

constexpr int kSigSet = 0;
constexpr int kSigAdd = 1;
constexpr int kCmpEq = 0, kCmpNe = 1, kCmpGt = 2, kCmpGe = 3, kCmpLt = 4, kCmpLe = 5;
constexpr int kSigStrideU64 = 16;  // 128-byte signal slots
constexpr uint32_t kErrTimeout = 1u;
constexpr uint32_t kErrCounts = 2u;    // AllToAll: a sender's counts were unusable
constexpr uint32_t kErrOverflow = 4u;  // AllToAll: a destination received more rows than it holds
constexpr int kSyncXcd = 0;    // producers and consumers of a stream share one XCD's L2
constexpr int kSyncAgent = 1;  // device-wide release/acquire (L2 write-back / invalidate)
constexpr int kThreads = 256;      // workgroup size of every copy kernel
constexpr int kNumXcd = 8;         // XCDs of an MI355X: at most this many stream groups
// queue words: per group a claim counter and a take-over counter, then a mask
// of groups whose queue is fully claimed, then one spare word
constexpr int kQueueSlots = 2 * kNumXcd + 2;
// reset flags of the combine's in-launch signal reset (slice 0, after the queue
// words): flag k holds the tag of the last launch whose zeroing workgroup k
// finished; never cleared by that reset itself
constexpr int kResetFlags = 64;

// Arguments of the signal-pipelined persistent combine.
struct PipeArgs {
    uint8_t* base;      // heap base (slice 0)
    int64_t stride;     // slice stride, bytes
    int64_t in_off;     // symmetric byte offsets of in, out, staging ring, signals
    int64_t out_off;
    int64_t stg_off;
    int64_t sig_off;
    uint32_t* err;      // device error word of the heap
    uint64_t* stamps;   // optional per-unit completion clock
    uint64_t timeout;   // spin timeout, device clock ticks
    int64_t S, H, D;    // problem
    int64_t BS, TH, TD; // tile (tokens, heads, d elements)
    int32_t W, e;       // ranks, element bytes
    int32_t nbs, nhb, ndb;     // signal-tile blocks along S, H, D
    int32_t MH;         // head blocks moved together (one piece / unit spans MH signal tiles)
    int32_t nmhb;       // merged head blocks: ceil(nhb / MH)
    int32_t R;          // ring depth (S-blocks)
    int32_t protocol;   // kSigSet | kSigAdd
    int32_t NG;         // stream groups (one per XCD when sync == kSyncXcd)
    int32_t nstreams;   // streams in total; group g owns [g*nstreams/NG, (g+1)*nstreams/NG)
    int32_t KB;         // streams of a group in flight together (a stream batch)
    int32_t sync;       // kSyncXcd | kSyncAgent
    int32_t csplit;     // consumer work items per unit (each copies one contiguous part)
    int32_t lookahead;  // tiles whose pieces precede a tile's consumer items in the queue
                        // (-1: all pieces first)
    int64_t regionA;    // data-signal slots per slice (credits follow)
    int64_t regionB;    // ring hand-back slots per slice (work counters follow, slice 0)
    int64_t ring_bytes; // staging bytes per slice
    int32_t direct;     // 1: pieces go straight to out_j, no staging
    int32_t PR;         // tokens per piece (direct mode: <= BS; staged modes: BS)
    int32_t nsub;       // pieces per full S-block and source (ceil(BS / PR)); > 1: the
                        // pieces of a tile count their arrivals in region B
    int32_t dyn;        // 1: persistent workgroups claim pieces / units from a counter
    int64_t claim_off;  // absolute byte offset of that counter (slice 0, the spare queue word)
    int32_t rows;       // 1 (with direct): row units -- whole rows of out_j, every source
    int32_t KU;         // row units: tokens per unit (a unit never straddles S-blocks)
    int32_t upb;        // row units per full S-block: ceil(BS / KU)
    int32_t ru;         // row units: rounds in flight per lane (4 or 8)
    int64_t nunits;     // row units in total
    int32_t inverse;    // 1: the dispatch (the combine's inverse map), direct mode only
    int32_t bulk;       // 1: staging in the two-phase layout [W][S][H][D], no ring
    int32_t pull;       // 1 (with bulk): the staging lives in the sender's slice, [j][S][H][D]
    int32_t straggler;  // delayed source rank or -1
    uint32_t delay;     // busy-loop base n0
    uint64_t seed;      // SplitMix64 seed of the delays
    int64_t units_per_dest;  // consumer units per destination (timestamps row)
    // in-launch signal reset (direct mode): reset_nz extra workgroups, the launch's
    // lowest block ids (before the piece_grid workgroups that move data), zero
    // slots [0, reset_slots) of every slice (reset_chunk each) and their share of
    // the timestamps (stamp_chunk each), then set their reset flag to reset_tag;
    // 0 = no in-launch reset
    uint64_t reset_tag;
    int32_t reset_nz;
    int32_t piece_grid;
    int64_t reset_slots, reset_chunk, stamp_chunk;
    int64_t flag_off;   // symmetric offset of reset flag 0 (used in slice 0)
};

// Arguments of the two-phase combine's two launches.
struct TwoPhaseArgs {
    uint8_t* base;
    int64_t stride;
    int64_t in_off, out_off, stg_off;
    int64_t S, H, D;
    int32_t W, e;
};

}  // namespace ra2a
