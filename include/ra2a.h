/*
 * ra2a -- Reverse All2All (EP-MoE combine) over a symmetric heap, MI355X (gfx950).
 *
 * C ABI of libra2a.so.  Plain pointers and sizes only; every call returns an int
 * status (RA2A_OK or a negative RA2A_E* code) unless stated otherwise, and no C++
 * exception crosses this boundary.  ra2a_last_error() returns a thread-local
 * message describing the most recent failure on the calling thread.
 *
 * Simulated ranks.  W ranks live on one GPU as W equal slices of one device
 * allocation (the symmetric heap).  Slice r is rank r's heap; a buffer has the
 * same offset inside every slice, so rank r's copy of a buffer whose slice-0
 * address is p is p + r * stride.  "Remote" stores are stores into another
 * slice of the same HBM.
 *
 * Streams.  `stream` arguments are hipStream_t values passed as void*; NULL is
 * the default stream.  Calls that take a stream only enqueue work: errors found
 * before enqueueing are returned at once, asynchronous device-side errors (a
 * bounded wait that timed out) are reported by ra2a_check().
 *
 * Device pointers.  Unless stated otherwise pointers are device addresses inside
 * one heap created by ra2a_symm_heap_create (found by address; no handle is
 * passed to the combine).  The library never frees memory it did not allocate.
 */
#ifndef RA2A_H_
#define RA2A_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes -------------------------------------------------------- */
#define RA2A_OK 0
#define RA2A_EINVAL (-1)       /* bad argument (range, alignment, overlap, heap) */
#define RA2A_ENOMEM (-2)       /* heap slice or device memory exhausted */
#define RA2A_EHIP (-3)         /* a HIP runtime call failed (message has the HIP error) */
#define RA2A_ETIMEOUT (-4)     /* a bounded device-side wait gave up */
#define RA2A_EUNSUPPORTED (-5) /* combination not implemented */
#define RA2A_EDATA (-6)        /* a device-side check of device-resident data failed */

/* ---- signal operations ----------------------------------------------------
 * "Distributed Architecture Design", section 2.3 (SignalOp SET / ADD) and the
 * HyperParallel RFC, section 四 (shmem_signal_op).  The two pages number them
 * differently (1/2 versus 0/1); the ABI uses these names, with SET = 0.       */
#define RA2A_SIG_SET 0 /* signal := value */
#define RA2A_SIG_ADD 1 /* signal += value (64-bit, wrapping) */

/* ---- wait predicates ------------------------------------------------------
 * "Distributed Architecture Design", section 6.3: eq, ne, gt, ge, lt, le
 * (unsigned 64-bit comparison of the signal against the value).             */
#define RA2A_CMP_EQ 0
#define RA2A_CMP_NE 1
#define RA2A_CMP_GT 2
#define RA2A_CMP_GE 3
#define RA2A_CMP_LT 4
#define RA2A_CMP_LE 5

/* ---- element types: the combine copies raw elements, only the size matters */
#define RA2A_U8 0   /* 1 byte  */
#define RA2A_BF16 1 /* 2 bytes */
#define RA2A_F16 2  /* 2 bytes */
#define RA2A_I32 3  /* 4 bytes */
#define RA2A_F32 4  /* 4 bytes */
#define RA2A_I64 5  /* 8 bytes */
#define RA2A_F64 6  /* 8 bytes */

/* One signal per 128-byte L2 line, so concurrent updates of neighbouring
 * signals never share a line ("Wait/Notify Optimization": one cache line per
 * signal slot; 128 B is gfx950's L2 line).  A signal array of n slots spans
 * n * RA2A_SIG_STRIDE_BYTES bytes; slot i is the uint64_t at byte
 * i * RA2A_SIG_STRIDE_BYTES.                                                   */
#define RA2A_SIG_STRIDE_BYTES 128
#define RA2A_SIG_STRIDE_U64 16

typedef struct ra2a_heap ra2a_heap_t;

/* ======================================================================== *
 * Symmetric heap ("Distributed Architecture Design", sections 5.1-5.3;      *
 * HyperParallel RFC, section 二).                                           *
 * ======================================================================== */

/* Create a heap of `world` slices of at least `slice_bytes` bytes each (the
 * slice stride is slice_bytes rounded up to 2 MiB) with one hipMalloc on the
 * current device.  The heap owns the memory; ra2a_symm_heap_destroy frees it.
 * Errors: EINVAL (world < 1 or > 4096, slice_bytes == 0, out == NULL), ENOMEM,
 * EHIP.                                                                        */
int ra2a_symm_heap_create(int world, size_t slice_bytes, ra2a_heap_t **out);

/* Adopt caller-owned device memory as a heap: `world` slices of `stride` bytes
 * starting at `base` (base and stride multiples of 256).  The caller keeps
 * ownership and must keep the memory alive until ra2a_symm_heap_destroy, which
 * then only unregisters the heap.  Errors: EINVAL (alignment, NULL, world out
 * of range, range overlapping a live heap), EHIP.                              */
int ra2a_symm_heap_attach(void *base, int world, size_t stride, ra2a_heap_t **out);

/* Free a heap and everything allocated from it (an attached heap's memory is
 * left to its owner).  Waits for the device first.  Passing NULL is a no-op
 * returning RA2A_OK.                                                            */
int ra2a_symm_heap_destroy(ra2a_heap_t *heap);

/* Symmetric allocation: reserve `bytes` at the same offset in every slice
 * (bump allocator; `align` a power of two, 0 = 4096 for 4 KiB or more, else
 * 256).  The same-size, same-order rule of collective allocation holds
 * trivially.  Returns the offset from the start of a slice.  Memory is not
 * initialised.  Placement matters for the combine's HBM traffic: with the
 * W=8, S=512, H=16, D=128 bf16 buffers at offsets off the 4 KiB grid it ran
 * 2-3 % slower than at 4 KiB-aligned ones, which were within 0.5 % of 1 or
 * 2 MiB-aligned ones.
 * Errors: EINVAL, ENOMEM (slice exhausted).                                     */
int ra2a_symm_malloc(ra2a_heap_t *heap, size_t bytes, size_t align, size_t *sym_offset);

/* Base address, slice stride (bytes) and world size; any output may be NULL. */
int ra2a_symm_heap_info(const ra2a_heap_t *heap, void **base, size_t *stride, int *world);

/* The heap containing device address `ptr`, or NULL. */
ra2a_heap_t *ra2a_symm_heap_find(const void *ptr);

/* symm_at ("Distributed Architecture Design", section 5.3): the address of
 * ptr's twin in rank `rank`'s slice, base + rank*stride + ((ptr - base) mod
 * stride).  Pure host arithmetic, no device access.  Returns NULL if ptr is
 * outside the heap or rank is outside [0, world).                              */
void *ra2a_symm_at(const ra2a_heap_t *heap, const void *ptr, int rank);

/* Timeout of every bounded device-side wait issued for this heap, in
 * microseconds (default 5,000,000).  0 restores the default.                   */
int ra2a_symm_heap_set_spin_timeout(ra2a_heap_t *heap, uint64_t timeout_us);

/* ======================================================================== *
 * One-sided primitives (HyperParallel RFC, sections 四 and 六; push mode,  *
 * section 5.1).                                                             *
 * ======================================================================== */

/* put_with_signal: copy `bytes` from `src` (any device memory) to
 * symm_at(dst_sym, target_rank), make the data visible device-wide, then apply
 * `sig_op` with `value` to symm_at(sig_sym, target_rank).  The signal is never
 * updated before the copy is complete and visible (fence before signal).
 * Asynchronous on `stream`.  dst_sym and sig_sym must lie in `heap`, sig_sym
 * 8-byte aligned; the destination range must not cross the end of the slice
 * and must not overlap src.  bytes may be 0 (signal only).
 * Errors: EINVAL, EHIP.                                                         */
int ra2a_put_with_signal(const ra2a_heap_t *heap, void *dst_sym, const void *src, size_t bytes,
                         uint64_t *sig_sym, uint64_t value, int sig_op, int target_rank,
                         void *stream);

/* put: the data part of put_with_signal alone (no signal).  Same rules.        */
int ra2a_put(const ra2a_heap_t *heap, void *dst_sym, const void *src, size_t bytes,
             int target_rank, void *stream);

/* get: the pull direction ("Push 模式与 Pull 模式", section 5.2; shmem_get in
 * section 四): copy `bytes` from symm_at(src_sym, source_rank) to `dst` (any
 * device memory).  Same range and overlap rules as put.                        */
int ra2a_get(const ra2a_heap_t *heap, void *dst, const void *src_sym, size_t bytes,
             int source_rank, void *stream);

/* signal_op: `sig_op` with `value` on symm_at(sig_sym, target_rank), ordered
 * after all earlier work on `stream`.  Errors: EINVAL, EHIP.                    */
int ra2a_signal_op(const ra2a_heap_t *heap, uint64_t *sig_sym, uint64_t value, int sig_op,
                   int target_rank, void *stream);

/* wait_for_signal: block `stream` until (*sig  cmp_op  cmp_value) holds
 * (acquire: device memory written before the matching signal is visible to
 * work enqueued after the wait).  Non-consuming: the signal is not modified,
 * so several waiters on one slot are safe.  Bounded: after the heap's spin
 * timeout the wait gives up, the heap's error word is set and the stream
 * continues; ra2a_check() then returns ETIMEOUT.  sig must lie in `heap`.
 * Errors: EINVAL, EHIP.                                                         */
int ra2a_wait_signal(const ra2a_heap_t *heap, const uint64_t *sig, uint64_t cmp_value,
                     int cmp_op, void *stream);

/* Zero `n_slots` signal slots (RA2A_SIG_STRIDE_BYTES apart) starting at
 * symm_at(sig_sym, r) for every rank r of the heap (the host-side reset before
 * a launch, "Reverse All2All (EP MoE Distributed Kernel)", "Host Side
 * Modifications").  Uses a kernel, not a memset node.  Errors: EINVAL, EHIP.    */
int ra2a_signal_reset(const ra2a_heap_t *heap, uint64_t *sig_sym, int64_t n_slots,
                      void *stream);

/* ======================================================================== *
 * Reverse All2All ("Reverse All2All (EP MoE Distributed Kernel)").          *
 *                                                                           *
 * For W ranks, rank r's input in_r has shape (S*W, H, D) and rank j's output *
 * out_j has shape (S, H*W, D), both row-major, elements of the size fixed   *
 * by `dtype`:                                                                *
 *                                                                           *
 *     out_j[s, r*H + h, d] = in_r[j*S + s, h, d]                            *
 *                                                                           *
 * (section "Reverse All2All Operator Semantics"; column r*H + h and row      *
 * j*S + s as in the MTE listing).  `in`, `out` and `signals` are addresses   *
 * inside one heap with world == W; rank r's buffers are their twins in slice *
 * r.  Elements are moved as raw bytes, so the result is bit-exact for every  *
 * type (NaN payloads, -0.0 and subnormals included).  in and out must not    *
 * overlap in any slice; each of in/out must fit inside its slice.           *
 * ======================================================================== */

/* Signalling protocols of the pipelined combine (ra2a_opts_t.protocol). */
#define RA2A_PROTO_ADD 1 /* push mode: W adds per tile, wait for W (default) */
#define RA2A_PROTO_SET 2 /* one SET per (source, tile) piece, wait for 1 */

/* Which map a launch performs (ra2a_opts_t.direction). */
#define RA2A_DIR_COMBINE 0  /* out_j[s, r*H + h, d] = in_r[j*S + s, h, d] */
#define RA2A_DIR_DISPATCH 1 /* out_r[j*S + s, h, d] = in_j[s, r*H + h, d] (the inverse) */

/* Where producers put their pieces (ra2a_opts_t.mode). */
#define RA2A_MODE_DIRECT 1 /* one piece per (source, tile), straight into out_j */
#define RA2A_MODE_STAGED 2 /* through a staging ring in slice j, reordered by consumers */
#define RA2A_MODE_BULK 3   /* two-phase layout with fine-grained signals (see below) */
#define RA2A_MODE_PULL 4   /* senders stage in their own slice, receivers pull (see below) */
#define RA2A_MODE_ROWS 5   /* row units: whole rows of out_j, all sources */

/* Work-queue words the pipelined combine keeps after the hand-back counters
 * (used in slice 0 only, staged mode only; direct mode leaves them 0): per
 * stream group (up to 8) a claim counter and a take-over counter, then a mask
 * of fully claimed groups and a spare word.                                   */
#define RA2A_QUEUE_SLOTS 18

/* Reset flags the pipelined combine keeps after the work-queue words (slice 0
 * only): in direct mode the signal reset runs inside the combine launch
 * (ra2a_rev_all2all), and zeroing workgroup k publishes its share by setting
 * flag k to the launch's tag.  They are never cleared by that reset.         */
#define RA2A_RESET_FLAGS 64

/* Tiling, protocol and launch options of the signal-pipelined kernel; a zeroed
 * struct (with straggler_rank = -1) means every default.                     */
typedef struct ra2a_opts {
    int64_t tile_s;     /* tokens per tile (default min(S, 64)) */
    int64_t tile_h;     /* heads per tile (default 1) */
    int64_t tile_d;     /* elements of D per tile (default D) */
    int32_t protocol;   /* RA2A_PROTO_ADD (or 0, the default): one signal per tile (j,
                         * s-block, head block, d block), each of the W sources adds 1, the
                         * consumer waits for W.  RA2A_PROTO_SET: one signal per piece
                         * (source r, tile), set to 1; the consumer waits for each piece. */
    int32_t ring;       /* staged mode: staging ring depth in S-blocks (default 8; >= the
                         * number of S-blocks means no slot is reused) */
    int32_t wg_per_cu;  /* persistent workgroups per compute unit (default 2; 1 for row
                         * units, and when per-source pieces are claimed dynamically --
                         * 8 or more per compute unit; capped at the kernel's occupancy).
                         * Row units always take a static schedule. */
    int32_t lookahead;  /* staged mode: tiles whose pieces are queued ahead of a tile's
                         * consumer work (0: default -- half of what the ring allows, or
                         * every piece first when no slot is reused; -1: every piece
                         * first); always capped so that no wait points forward */
    int32_t straggler_rank;   /* source slice whose producers are delayed, -1 = none */
    uint32_t straggler_delay; /* busy-wait base n0: before each of its pieces the
                               * delayed source waits n0 + u ticks of the 100 MHz
                               * device clock, u uniform in [0, n0] from SplitMix64
                               * (Steele, Lea and Flood 2014) indexed by the piece */
    uint64_t straggler_seed;  /* seed of that SplitMix64 sequence */
    uint64_t *timestamps;     /* optional device array, zeroed by the caller: for each
                               * destination slice j and data-signal slot u, the device
                               * real-time clock at which that signal tile was complete,
                               * at timestamps[j * tile_slots + u] (direct mode: the
                               * latest of its pieces' signals; staged mode: the end of
                               * its consumer copy) */
    int32_t mode;             /* 0: the default -- RA2A_MODE_ROWS when one source's run
                               * of a token row, H*D*e bytes, is at most 8 KiB and
                               * divides or is a multiple of 4096, and none of a
                               * delayed straggler source, head_merge or piece_rows is
                               * set; RA2A_MODE_DIRECT otherwise (the combine and the
                               * dispatch alike).
                               * RA2A_MODE_ROWS: each work unit fills unit_rows whole
                               * token rows of out_j (the W sources' runs of H*D elements,
                               * one contiguous range of out_j; W contiguous ranges of
                               * the inputs, read source after source) and adds 1 to its
                               * S-block's arrival counter (region B: one per S-block).
                               * Under ADD with W a multiple of the block's unit count
                               * nub, each unit also adds W / nub to every signal tile of
                               * its block once its rows are released (a tile reaches W
                               * when all nub units have stored); otherwise the unit that
                               * completes the block's count marks every signal tile of
                               * the block complete (ADD W, or SET 1 on each (tile,
                               * source) slot).  Either way the final values are the ones
                               * W pieces would leave.  The dispatch's unit is the mirror
                               * image: source j's unit_rows rows of in_j, read whole,
                               * give each destination r one contiguous range (rows
                               * j*S + s0 .. of out_r), and the unit that completes the
                               * block's count (region B of slice j) sets the block's
                               * (tile, j) slot in every destination's slice.  Not with a
                               * delayed straggler source (every unit carries all
                               * sources).
                               * RA2A_MODE_DIRECT: producers store each piece (one
                               * source's rows of a tile, or a part of them: piece_rows)
                               * straight into its final place in out_j (a symmetric
                               * buffer) and signal the tile.
                               * Both direct modes: no ring, no consumer copy, no
                               * hand-back, no work queue (a static schedule); the data
                               * is released device-wide before a signal, so a tile
                               * whose signal reads its final value (W under ADD, 1 on
                               * each of its slots under SET) is complete in out_j and
                               * visible to any reader on the device that acquires the
                               * signal (ra2a_wait_signal, or a later kernel), even
                               * while the launch still runs.
                               * RA2A_MODE_STAGED: producers store into slice j's staging
                               * ring (the pages' window layout), consumers wait, copy
                               * ring -> out_j and hand the ring slot back.
                               * RA2A_MODE_BULK ("UDMA Optimized Implementation", section
                               * "Wait/Notify Optimization"): the two-phase exchange with
                               * per-(S-block, sender) signals instead of a barrier.  Source
                               * r copies its segment in_r[j*S + b*tile_s ..] straight
                               * into slice j's staging [W][S][H][D] at [r][b*tile_s ..]
                               * (the input's own layout) and sets slot (b, r) of region A
                               * (slot b*W + r with whole-row tiles; the SET layout is
                               * forced); a consumer waits only for its sender's slot, then
                               * reorders that block into out_j.  No ring, no hand-back
                               * (region B is empty).  Staging of 4 GiB or more per slice
                               * needs agent_sync (EINVAL otherwise).
                               * RA2A_MODE_PULL (HyperParallel RFC, section 5.2, pull
                               * mode): the sender first copies its segment for j into its
                               * OWN slice's staging [W][S][H][D] at [j][b*tile_s ..] (the
                               * same offset as its input rows) and sets slot (b, r) in
                               * slice j; the receiver waits for that slot, then reads the
                               * block from the sender's slice and reorders it into out_j.
                               * Signals, staging size (workspace_bytes) and limits as
                               * RA2A_MODE_BULK; slice r's copy of the staging holds
                               * sender r's outgoing segments instead of receiver j's
                               * incoming ones. */
    int32_t consumer_split;   /* staged mode: consumer work items sharing one unit, each
                               * copying a contiguous part (default: one per 128 KiB;
                               * at most 4096) */
    int32_t skip_reset;       /* 1: the caller has already zeroed every signal slot
                               * (ra2a_signal_reset on the same stream); the combine
                               * zeroes none (the timestamps, if any, it still zeroes) */
    int32_t stream_batch;     /* tile streams of one XCD in flight together (default: as
                               * many as fit about 2 MiB of staging ring) */
    int32_t agent_sync;       /* 1: synchronise producers and consumers with device-wide
                               * release/acquire (L2 write-back / invalidate) instead of
                               * the XCD-local protocol, and let every workgroup serve
                               * every stream group */
    int32_t head_merge;       /* signal tiles of adjacent head blocks moved together by one
                               * piece / unit (each keeps its own signal); default, when a
                               * tile spans all of D: runs of up to 4 KiB, halved until the
                               * call has at least 512 pieces (direct modes; their pieces
                               * above 128 KiB then move in parts, see piece_rows) or 1024
                               * (staged modes) */
    int32_t separate_reset;   /* 1: zero the signals with a launch of their own before the
                               * combine's, also in direct mode (0, the default: direct
                               * mode zeroes them inside the combine launch) */
    int32_t direction;        /* RA2A_DIR_COMBINE (0, the default) or RA2A_DIR_DISPATCH (the
                               * inverse map; see ra2a_all2all_dispatch) */
    int32_t unit_rows;        /* RA2A_MODE_ROWS: tokens per row unit (0: the default,
                               * max(1, 262144 / (W*H*D*e)) -- about 256 KiB of output --
                               * or max(1, 524288 / (W*H*D*e)) when H*D*e >= 4096 and the
                               * call then still has at least 256 units; always capped
                               * at tile_s, and a unit never straddles two S-blocks) */
    int32_t piece_rows;       /* RA2A_MODE_DIRECT: tokens per piece, at most tile_s (0:
                               * the default -- a tile's rows of one source in one piece
                               * up to 128 KiB, else cut into ceil(bytes / 128 KiB)
                               * pieces of equal token counts).  With more than one
                               * piece per tile and source, each tile counts its
                               * pieces' arrivals in region B and the piece that
                               * completes it signals it (ADD W, or SET 1 per source) */
    int32_t reserved[1];      /* must be zero */
} ra2a_opts_t;

/* Number of signal slots the combine needs per slice: `tile_slots` data
 * signals (region A: ADD, one per (s-block, head block, d block) in that
 * order; SET, one per (s-block, head block, d block, source r)), then
 * `credit_slots` counters (region B; staged mode: ring hand-back counters, ADD
 * [ring slot][merged head block][d block], SET [ring slot][merged head
 * block][d block][source], where a merged head block is head_merge adjacent
 * head blocks; RA2A_MODE_ROWS: one arrival counter per S-block; 0 in the
 * other modes), then `queue_slots` control words
 * (RA2A_QUEUE_SLOTS work-queue words, then RA2A_RESET_FLAGS reset flags; 0 for
 * an empty problem).  The
 * `signals` array of a combine must hold the sum of the three in every slice.
 * opts may be NULL; any output pointer may be NULL.                          */
int ra2a_rev_all2all_signal_slots(int W, int64_t S, int64_t H, int64_t D, int dtype,
                                  const ra2a_opts_t *opts, int64_t *tile_slots,
                                  int64_t *credit_slots, int64_t *queue_slots);

/* The tiling, mode and work a combine with these options resolves to (no GPU
 * needed): what the defaults chose, so that callers and tests can predict the
 * signal arrays.  The launch adds the schedule, which depends on the device:
 * per-source pieces are claimed dynamically (a counter in the last
 * RA2A_QUEUE_SLOTS word, slice 0, ending at work_items) when there are at least
 * 8 per compute unit, else walked statically; row units are always walked
 * statically (that word stays 0).                                             */
typedef struct ra2a_plan {
    int32_t mode;            /* RA2A_MODE_DIRECT, _ROWS, _STAGED, _BULK or _PULL */
    int32_t protocol;        /* RA2A_PROTO_ADD or RA2A_PROTO_SET: the signal layout used */
    int64_t tile_s, tile_h, tile_d;
    int32_t head_merge;      /* signal tiles of adjacent head blocks moved together */
    int32_t piece_rows;      /* direct mode: tokens per piece (tile_s in the staged modes) */
    int32_t pieces_per_tile; /* direct mode: pieces per tile and source, ceil(tile_s /
                              * piece_rows); > 1 means region B holds arrival counters */
    int32_t unit_rows;       /* RA2A_MODE_ROWS: tokens per row unit (0 otherwise) */
    int64_t tile_slots, credit_slots, queue_slots; /* as ra2a_rev_all2all_signal_slots */
    int64_t work_items;      /* direct modes: pieces or row units per launch (0 otherwise) */
    size_t workspace_bytes;  /* as ra2a_rev_all2all_workspace_bytes (pipelined) */
} ra2a_plan_t;

int ra2a_rev_all2all_plan(int W, int64_t S, int64_t H, int64_t D, int dtype,
                          const ra2a_opts_t *opts, ra2a_plan_t *plan);

/* Staging bytes per slice the library reserves from the heap on first use
 * (pipelined: the ring; two_phase != 0: a full (W, S, H, D) staging area).     */
int ra2a_rev_all2all_workspace_bytes(int W, int64_t S, int64_t H, int64_t D, int dtype,
                                     const ra2a_opts_t *opts, int two_phase, size_t *bytes);

/* The combine with the signal-pipelined persistent kernel and default options
 * (row units, RA2A_MODE_ROWS).  Every signal slot and work-queue word is zeroed
 * before any producer of the launch signals ("Host Side Modifications").  In
 * the direct modes one launch does both: its lowest-numbered workgroups zero the
 * slots and publish their share through the reset flags (dispatched first, so
 * no occupancy is needed beside them), and the persistent workgroups walk the
 * row units (or, RA2A_MODE_DIRECT, the producer pieces) on a static schedule:
 * each copies its rows with 16-byte stores straight into out_j, releases them
 * device-wide and, once the reset flags carry this launch's tag, counts or
 * signals its tiles.  (Staged, bulk and pull modes, or separate_reset: the
 * reset is a launch of its own before the combine's.)  In staged
 * mode they take tasks from one work queue per XCD: producer pieces into the
 * staging ring, and consumer work, which waits until its tile's signal is
 * complete, copies the ring into out_j and hands the ring slot back.
 * Afterwards every region-A slot holds W (ADD) or 1 (SET), and every region-B
 * slot the number of consumer work items that used it (staged) or the number
 * of row units of its S-block (row units).  Staging (staged, bulk and pull
 * modes) comes from the heap (see workspace_bytes) and is one area per heap,
 * shared by every such call on the heap whatever its stream: calls that use
 * staging on one heap must be ordered (one stream, or events between them),
 * else they race on it.  Under stream capture (a HIP graph)
 * the reset is always a launch of its own, so replays stay correct; make one call
 * outside capture first (the first call on a heap allocates its error word and
 * probes the device's XCDs).
 * Errors: EINVAL, ENOMEM (heap too small for the staging ring), EHIP.           */
int ra2a_rev_all2all(const void *in, void *out, uint64_t *signals, int W, int64_t S, int64_t H,
                     int64_t D, int dtype, void *stream);

/* Same, with explicit tiling / protocol / straggler options (opts may be NULL). */
int ra2a_rev_all2all_ex(const void *in, void *out, uint64_t *signals, int W, int64_t S,
                        int64_t H, int64_t D, int dtype, const ra2a_opts_t *opts, void *stream);

/* Forward All2All (dispatch), read as the exact inverse of the combine
 * ("Reverse All2All (EP MoE Distributed Kernel)", sections "Reverse All2All
 * Operator Semantics" and "EP MoE Scenario": the dispatch sends tokens to the
 * experts' ranks and the combine brings the outputs back, so a combine after a
 * dispatch returns every element to its place).  Rank j's input `in` (slice j)
 * is (S, H*W, D); rank r's output `out` (slice r) is (S*W, H, D):
 *     out_r[j*S + s, h, d] = in_j[s, r*H + h, d].
 * Same buffers, heap, tiling options and in-launch reset as the direct-mode
 * combine: the signal tile (source j's S-block b, head block, d block) of
 * destination r has one slot per source (the SET layout,
 * ra2a_rev_all2all_signal_slots with direction = RA2A_DIR_DISPATCH), and each
 * ends at 1.  Row units and per-source pieces as for the combine (the same
 * default rule); staged mode is rejected (EINVAL).  _ex takes the combine's
 * options (direction is forced to RA2A_DIR_DISPATCH).
 * Errors: EINVAL, EHIP.                                                         */
int ra2a_all2all_dispatch(const void *in, void *out, uint64_t *signals, int W, int64_t S,
                          int64_t H, int64_t D, int dtype, void *stream);
int ra2a_all2all_dispatch_ex(const void *in, void *out, uint64_t *signals, int W, int64_t S,
                             int64_t H, int64_t D, int dtype, const ra2a_opts_t *opts,
                             void *stream);

/* The two-phase variant ("UDMA Optimized Implementation": "Two-Phase Data
 * Copy"): phase 1 copies every contiguous (S, H, D) segment in_r[j*S, (j+1)*S)
 * into slot r of rank j's full-size staging area; stream order between the two
 * launches is the barrier; phase 2 reorders staging into out_j.  `signals` is
 * not used and may be NULL.  The staging area is the heap's (shared by every
 * two-phase call on the heap: order them on one stream).
 * Errors: EINVAL, ENOMEM, EHIP.                                                 */
int ra2a_rev_all2all_two_phase(const void *in, void *out, uint64_t *signals, int W, int64_t S,
                               int64_t H, int64_t D, int dtype, void *stream);

/* ---- AllGather + GEMM ---------------------------------------------------- */
/* ("Triton-distributed Semantics", sections "Producer-Consumer Model" and
 * "AllGather + GEMM Overlapping"; HyperParallel RFC, section 十
 * fused_all_gather_matmul, read as C = gather(A) @ B with no reduction.)
 *
 * W row shards A_w (m_local x K bf16, row-major; shard w is `a_shards`' twin
 * in slice w) are gathered into G (W*m_local x K bf16; `gathered`'s twin in
 * slice `rank`, shard w at rows [w*m_local, (w+1)*m_local)), and
 *     C = G @ B      (B: K x N bf16 row-major, C: W*m_local x N bf16 row-major)
 * with fp32 accumulation on the matrix cores and bf16 output rounded to
 * nearest even.  One persistent launch: every tile of `tile_rows` rows of a
 * shard is copied in parts into G and signalled (SET 1 on its slot once all
 * parts are in); each 256 x 256 output tile waits only for the tiles covering
 * its rows.  Signals live in slice `rank`: W*ntiles tile signals, then W*ntiles
 * part counters, then RA2A_QUEUE_SLOTS queue words (ntiles =
 * ceil(m_local / min(tile_rows, m_local))); ra2a_ag_gemm_signal_slots gives
 * the three counts.  Afterwards every tile signal holds 1 and every counter
 * its tile's number of parts.  `b` and `c` are device pointers the caller owns
 * (16- and 2-byte aligned; they must not overlap each other or the heap
 * buffers); the heap buffers must be 16-byte aligned and must not overlap.
 * K and N must be multiples of 8, and 512 * K below 2^32.  flags:
 * RA2A_AG_AGENT_SYNC (device-wide release/acquire instead of XCD-local),
 * RA2A_AG_SKIP_RESET (the caller has zeroed the signals on the stream),
 * RA2A_AG_B_TRANSPOSED (see below).
 * Errors: EINVAL (arguments), EUNSUPPORTED, EHIP; a device-side wait that gives
 * up surfaces through ra2a_check as ETIMEOUT.                                  */
#define RA2A_AG_AGENT_SYNC 1
#define RA2A_AG_SKIP_RESET 2
#define RA2A_AG_B_TRANSPOSED 4 /* `b` holds B^T (N x K row-major); otherwise the
                                  library transposes B into a workspace it owns
                                  (hipMalloc'd once per heap, freed with it).  That
                                  workspace is one per heap: calls on one heap
                                  with different B must be ordered on one stream,
                                  and a call that needs it larger synchronizes the
                                  device to replace it, so make the first call
                                  with the largest B outside graph capture (or
                                  use ra2a_ag_gemm_noalloc) */

int ra2a_ag_gemm_signal_slots(int W, int64_t m_local, int tile_rows, int64_t *tile_slots,
                              int64_t *count_slots, int64_t *queue_slots);

int ra2a_ag_gemm(const void *a_shards, void *gathered, const void *b, void *c, uint64_t *signals,
                 int W, int rank, int64_t m_local, int64_t K, int64_t N, int tile_rows, int flags,
                 void *stream);

/* The same AllGather+GEMM for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * It calls no hipMalloc, hipFree or other allocating routine.  Arguments,
 * results and errors as ra2a_ag_gemm; the kernels are the same.  Differences:
 *   - B^T (unless RA2A_AG_B_TRANSPOSED) goes to a static device array of the
 *     library, 64 MiB per GPU (K * N * 2 bytes at most, EINVAL beyond), which
 *     each GPU the library runs on holds until the process ends;
 *   - the device error word is in that array too: ra2a_check on any heap of
 *     the device reports (and clears) a wait that gave up;
 *   - unless an earlier allocating call on the device has measured its XCDs,
 *     producers and consumers synchronise device-wide (as RA2A_AG_AGENT_SYNC).
 * Every call on one GPU shares that array, which keeps the last call's B^T:
 * calls that overlap in time on one GPU (other streams, other threads) race on
 * it; order them on one stream.  The first call on a device looks up the
 * array's address (once per device; make it outside graph capture).          */
int ra2a_ag_gemm_noalloc(const void *a_shards, void *gathered, const void *b, void *c,
                         uint64_t *signals, int W, int rank, int64_t m_local, int64_t K,
                         int64_t N, int tile_rows, int flags, void *stream);

/* Host check of the AllGather+GEMM work queues for a device of `num_xcd` XCDs
 * (no GPU needed): every part and GEMM tile queued exactly once, parts cover
 * each shard's rows once without straddling tiles, and every GEMM tile queued
 * after all parts of the tiles it waits for.  *tasks_per_group (may be NULL)
 * receives the queue length.  Returns EINVAL with a message on a violation.   */
int ra2a_debug_ag_gemm_plan(int W, int rank, int64_t m_local, int64_t K, int64_t N, int tile_rows,
                            int num_xcd, int64_t *tasks_per_group);

/* ---- GEMM + ReduceScatter -------------------------------------------------- */
/* (HyperParallel RFC, section 十 fused_matmul_reduce_scatter; "Triton-distributed
 * Semantics", section "GEMM + ReduceScatter Overlapping".)  output =
 * ReduceScatter(x1 @ x2): rank r holds x1_r (m x K) and x2_r (K x N); rank j
 * receives out_j = rows [j*m/W, (j+1)*m/W) of sum_r x1_r @ x2_r (m must be
 * divisible by W).  One persistent launch of tasks, each a 256 x 256 tile of
 * rank r's partial product for destination j.  The tasks of the W - 1 other
 * ranks store their tiles into j's receive area at slot r and SET the (tile, r)
 * signal in j's slice; rank j's own task keeps its tile in its accumulators,
 * waits for those W - 1 signals, adds the partials in rank order 0..W-1 (its
 * own in its place) in fp32, stores bf16 (round to nearest even) and SETs
 * (tile, j).  The signals order the tasks inside the launch; out_j is complete,
 * for any reader, when the launch is (stream order).  A partial is the fp32
 * accumulator tile of x1_r @ x2_r (one rounding in all, to bf16 at the end), or
 * with RA2A_RS_BF16_PARTIALS that
 * product as the bf16 tensor a framework's matmul returns (rounded to nearest
 * even, rank j's own too): half the receive area and its traffic, at the cost
 * of W more roundings, so that where the partials cancel the elementwise error
 * is no longer bounded by the result's magnitude but by 2^-8 * sum_r
 * |partial_r|.  Tasks for destination j visit the sources in a rotation
 * ((j + 1 + s) mod W at step s, so rank r works for rank (r - 1 - s) mod W and
 * j's own task comes last).  bf16 operands, fp32 accumulation.  Every wait is
 * bounded (ra2a_check reports RA2A_ETIMEOUT).                                */
#define RA2A_RS_AGENT_SYNC 1 /* device-wide release/acquire instead of the XCD-local protocol */
#define RA2A_RS_SKIP_RESET 2 /* the caller zeroed the signals; no reset launch */
#define RA2A_RS_BF16_PARTIALS 4 /* partials rounded to bf16 instead of kept in fp32 */

/* Sizes for (W, m, K, N): `tile_slots` = (output tiles of out_j) * W signal slots
 * per slice, then `queue_slots` (RA2A_QUEUE_SLOTS) queue words (slice 0); the
 * `signals` array must hold their sum per slice.  `partial_bytes` = bytes of the
 * receive area per slice: W slots of one 256 x 256 partial tile per output tile,
 * fp32, or bf16 if `flags` holds RA2A_RS_BF16_PARTIALS (the other flags do not
 * change the sizes); its layout is the library's own (the accumulators in the
 * order the matrix-core lanes hold them).  Any output pointer may be NULL.
 * Errors: EINVAL.                                                               */
int ra2a_gemm_rs_sizes(int W, int64_t m, int64_t K, int64_t N, int flags, int64_t *tile_slots,
                       int64_t *queue_slots, size_t *partial_bytes);

/* All five buffers are symmetric, inside one heap of W slices, at these
 * offsets in every slice (row-major, bf16 unless stated):
 *   x1      slice r: x1_r, m x K (16-byte aligned);
 *   x2t     slice r: x2_r transposed, N x K (16-byte aligned);
 *   partial slice j: the receive area, ra2a_gemm_rs_sizes' partial_bytes
 *           (16-byte aligned; scratch, its contents are the library's);
 *   out     slice j: out_j, m/W x N (8-byte aligned);
 *   signals slice j: ra2a_gemm_rs_sizes' slots at 128-byte spacing (8-byte aligned).
 * K must be a multiple of 8, and 512 * K below 2^32 (a tile's operand rows are
 * addressed with 32-bit offsets).  The signals are zeroed by a reset launch first
 * unless RA2A_RS_SKIP_RESET.  After the call every tile slot holds 1.  The
 * library owns the buffers until the stream reaches the end of the launch.
 * Errors: EINVAL (shapes, flags, alignment, overlap, a buffer outside the heap
 * or crossing the end of a slice, K too large, a receive area of 4 GiB or more),
 * EHIP.                                                                        */
int ra2a_gemm_rs(const void *x1, const void *x2t, void *partial, void *out, uint64_t *signals,
                 int W, int64_t m, int64_t K, int64_t N, int flags, void *stream);

/* Host check of the GEMM+ReduceScatter work queues for a device of num_xcd
 * XCDs: every (destination, tile, source) task once, and each receiver's task
 * (source == destination) after the W - 1 tasks it waits for.  tasks_per_group
 * (optional) receives the queue length.  Returns EINVAL with a message on a
 * violation.                                                                   */
int ra2a_debug_gemm_rs_plan(int W, int64_t m, int64_t K, int64_t N, int num_xcd,
                            int64_t *tasks_per_group);

/* ---- variable-size AllToAll (push) ------------------------------------------ */
/* (HyperParallel RFC, section 十, "AllToAll (Push mode)".)  The split-size
 * all-to-all: rank r's input is rows of row_bytes bytes cut, in destination
 * order, into segments of send_counts_r[j] rows; rank j receives the
 * concatenation, in source order r = 0 .. W-1, of the segments addressed to it.
 * As on the page, the ranks first exchange metadata -- each sender puts its
 * count into the destination's recv_counts and adds 1 to its count signal; each
 * destination, once that reads W, hands every sender the row where its segment
 * goes -- then every sender pushes its segments (in the rotation j = (r + t) mod
 * W, t = 0 .. W-1, cut into chunks of chunk_bytes), and each destination's
 * arrival signal accumulates to W.  One launch: the counts stay on the device,
 * with no host round trip between metadata and data.  W <= 32.                */
#define RA2A_A2V_SKIP_RESET 1 /* the caller zeroed the signals; no reset launch */

/* Signal slots per slice (at 128-byte spacing): 2W + 3.  Errors: EINVAL.      */
int ra2a_alltoallv_signal_slots(int W, int64_t *slots);

/* All five buffers are symmetric, inside one heap of W slices, at these
 * offsets in every slice:
 *   in          slice r: in_rows rows of row_bytes bytes (16-byte aligned);
 *   send_counts slice r: int64[W], rows rank r sends to each rank (8-byte aligned;
 *               device memory, read by the kernel);
 *   out         slice j: out_rows rows of row_bytes bytes (16-byte aligned);
 *   recv_counts slice j: int64[W + 1]: [r] = rows received from rank r, [W] = the
 *               total, written once every segment has arrived (8-byte aligned);
 *   signals     slice j: ra2a_alltoallv_signal_slots' slots (8-byte aligned).
 * chunk_bytes: bytes per data task (0: 44 KiB; else a positive multiple of 16).
 * The signals are zeroed by a reset launch first unless RA2A_A2V_SKIP_RESET.
 * Checked on the device (ra2a_check then reports RA2A_EDATA): a sender with a
 * negative count, or more rows in total than in_rows, sends nothing (its counts
 * read as 0); a segment that would run past out_rows is not copied.  Either way
 * every signal still completes, so nothing waits out a timeout.  Afterwards the
 * count and arrival signals of every slice read W.  The library owns the
 * buffers until the stream reaches the end of the launch.
 * Errors: EINVAL (shapes, flags, alignment, overlap, a buffer outside the heap
 * or crossing the end of a slice), EHIP.                                     */
int ra2a_alltoallv(const void *in, const int64_t *send_counts, void *out, int64_t *recv_counts,
                   uint64_t *signals, int W, int64_t row_bytes, int64_t in_rows, int64_t out_rows,
                   int64_t chunk_bytes, int flags, void *stream);

/* Host emulation (no GPU needed) of the AllToAll's work queue, run strictly in
 * queue order with the kernel's own decode: in[r] and out[j] are host arrays
 * of in_rows / out_rows rows, send_counts W x W (row r = rank r's counts),
 * recv_counts W x (W + 1), signals W x (2W + 3) final slot values, *err_word
 * receives the device error bits.  Returns EINVAL if a task would wait for one
 * queued after it or a segment's chunks are not each queued once; *tasks
 * (optional) receives the queue length.                                      */
int ra2a_debug_alltoallv_emulate(int W, int64_t row_bytes, int64_t in_rows, int64_t out_rows,
                                 int64_t chunk_bytes, const void *const *in,
                                 const int64_t *send_counts, void *const *out, int64_t *recv_counts,
                                 uint64_t *signals, uint32_t *err_word, int64_t *tasks);

/* ---- diagnostics --------------------------------------------------------- */

/* Wait for the device, then report and clear the heap's device error word:
 * RA2A_EDATA if a device-side data check failed (the AllToAll's counts),
 * RA2A_ETIMEOUT if a bounded wait gave up since the last check, RA2A_EHIP if
 * the device reported an error, else RA2A_OK.                                  */
int ra2a_check(const ra2a_heap_t *heap);

/* Host emulation of the signal-pipelined combine (no GPU needed): runs the
 * kernel's own piece / work-item address arithmetic for a device of `num_cus`
 * compute units with `blocks_per_cu` resident workgroups -- direct mode: every
 * piece of the static schedule; staged mode: each work queue strictly in
 * order -- on host copies of the heap.  in[r]
 * (rank r's input) and out[j] are host arrays of S*W*H*D elements; signals[j]
 * (optional, may be NULL) receives the final tile_slots + credit_slots +
 * queue_slots signal values of slice j (unstrided; the queue words are not
 * modelled and read 0).  Returns EINVAL with a message if any access would
 * leave its buffer, if a queue does not hold every task once, or if a wait
 * would not already hold when its task comes up in queue order (which would
 * let the kernel deadlock).  For checking the index arithmetic on a host; it
 * is not a CPU fallback.                                                       */
int ra2a_debug_emulate_pipelined(const void *const *in, void *const *out,
                                 uint64_t *const *signals, int W, int64_t S, int64_t H,
                                 int64_t D, int dtype, const ra2a_opts_t *opts, int num_cus,
                                 int blocks_per_cu);

/* Message for the most recent failure on this thread ("" if none). */
const char *ra2a_last_error(void);

/* ABI version (major * 10000 + minor * 100 + patch). */
int ra2a_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RA2A_H_ */
