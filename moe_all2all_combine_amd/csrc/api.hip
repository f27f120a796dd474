// C ABI of libra2a: symmetric heap, one-sided primitives and the Reverse All2All
// combine (declarations and contracts in include/ra2a.h).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <random>
#include <string>
#include <vector>

#include "ag_gemm_geom.h"
#include "combine_geom.h"
#include "common.h"
#include "launch.h"
#include "ra2a.h"

#define RA2A_API extern "C" __attribute__((visibility("default")))

struct ra2a_heap {
    int world = 0;
    size_t stride = 0;
    uint8_t* base = nullptr;
    int device = 0;
    size_t bump = 0;               // next free symmetric offset
    uint32_t* err = nullptr;       // device error word (library-owned, outside the heap)
    uint64_t timeout_us = 0;       // 0 = default
    bool owned = true;             // false: attached caller memory
    size_t ring_off = 0, ring_bytes = 0;   // cached staging ring (pipelined combine)
    size_t full_off = 0, full_bytes = 0;   // cached full staging (two-phase combine)
    void* bt_ws = nullptr;         // B^T workspace of the AllGather+GEMM (library-owned)
    size_t bt_bytes = 0;
    std::mutex mu;
};

namespace {

constexpr size_t kSliceAlign = size_t(2) << 20;
constexpr uint64_t kDefaultTimeoutUs = 5000000ull;
thread_local std::string g_err;
// The heap registry lives until the process ends (never destroyed: no exit
// handler can find it half torn down).
std::mutex& g_reg_mu = *new std::mutex;
std::vector<ra2a_heap*>& g_heaps = *new std::vector<ra2a_heap*>;

// Set when the library is unloaded at process exit.  From then on the HIP
// runtime, the profiler's hooks and torch's allocator may already be gone, so a
// heap destroyed that late frees host state only and leaves its device memory
// to the runtime (callers should close heaps before exit; the Python binding
// does so from an atexit hook).
std::atomic<bool> g_exiting{false};
__attribute__((destructor)) void mark_exiting() { g_exiting.store(true); }

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

// Set while an allocation-free entry point runs on this thread: the library's
// own allocations (error words, workspaces, the XCD probe) refuse to run then.
thread_local bool g_no_alloc = false;
struct NoAllocScope {
    NoAllocScope() { g_no_alloc = true; }
    ~NoAllocScope() { g_no_alloc = false; }
};

int no_alloc_refused(const char* what) {
    return fail(RA2A_EUNSUPPORTED, "internal: %s would allocate inside an allocation-free entry point",
                what);
}

int hip_fail(hipError_t e, const char* what) {
    return fail(RA2A_EHIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

int ok() {
    return RA2A_OK;
}

int elem_bytes(int dtype) {
    switch (dtype) {
        case RA2A_U8: return 1;
        case RA2A_BF16:
        case RA2A_F16: return 2;
        case RA2A_I32:
        case RA2A_F32: return 4;
        case RA2A_I64:
        case RA2A_F64: return 8;
        default: return 0;
    }
}

ra2a_heap* find_heap(const void* p) {
    const uint8_t* q = static_cast<const uint8_t*>(p);
    std::lock_guard<std::mutex> g(g_reg_mu);
    for (ra2a_heap* h : g_heaps)
        if (q >= h->base && q < h->base + h->stride * (size_t)h->world) return h;
    return nullptr;
}

bool in_heap(const ra2a_heap* h, const void* p) {
    const uint8_t* q = static_cast<const uint8_t*>(p);
    return h && q >= h->base && q < h->base + h->stride * (size_t)h->world;
}

size_t sym_offset(const ra2a_heap* h, const void* p) {
    return (size_t)(static_cast<const uint8_t*>(p) - h->base) % h->stride;
}

uint64_t timeout_ticks(const ra2a_heap* h) {
    int khz = 0;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess ||
        khz <= 0)
        khz = 100000;  // gfx9 real-time clock: 100 MHz
    const uint64_t us = h->timeout_us ? h->timeout_us : kDefaultTimeoutUs;
    return us * (uint64_t)khz / 1000ull;
}

// The device error word of a heap, allocated on first use (so that a heap can
// be attached and validated on a host without a GPU).
int ensure_err(ra2a_heap* h) {
    std::lock_guard<std::mutex> g(h->mu);
    if (h->err) return RA2A_OK;
    if (g_no_alloc) return no_alloc_refused("the heap's error word");
    void* ew = nullptr;
    hipError_t e = hipMalloc(&ew, 256);
    if (e == hipSuccess) e = hipMemset(ew, 0, 256);
    if (e != hipSuccess) {
        if (ew) (void)hipFree(ew);
        (void)hipGetLastError();
        return hip_fail(e, "error word allocation");
    }
    h->err = static_cast<uint32_t*>(ew);
    return RA2A_OK;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Default output bytes per row unit (RA2A_MODE_ROWS): the unit_rows default is
// max(1, kRowUnitBytes / (W*H*D*e)) tokens, at most the S-block -- or twice
// that when a source's run (H*D*e) is at least kRowWholeRun (a 4 KiB round of
// 256 lanes x 16 B lies in one run) and the call still has kRowUnitsMin units
// (one per compute unit of the 256 of gfx950).  Measured (bf16, tile_s 64,
// 256 KiB against 512 KiB units): W=8, S=512, H=16, D=128 47.8 against 47.1 us;
// W=16, S=256, H=16, D=128 96.1 against 91.8; W=8, S=1024, H=8, D=128 (2 KiB
// runs) 48.2 against 51.7; W=4, S=1024, H=16, D=128 (128 units) 27.5 against
// 31.6.
constexpr int64_t kRowUnitBytes = 256 << 10;
constexpr int64_t kRowWholeRun = 4 << 10;
constexpr int64_t kRowUnitsMin = 256;
// Mode 0 moves row units when one source's run of a token row (H*D*e bytes) is at
// most this and divides or is a multiple of the 4 KiB round (kRowWholeRun),
// per-source pieces otherwise.  Measured on gfx950 (bf16, tile_s 64, percent of
// 8 TB/s, row units against pieces): runs of 1 KiB (W=8, S=2048, H=4, D=128) 70
// against 57, 4 KiB (W=8, S=512, H=16, D=128) 72 against 69, 4 KiB at W=16 74
// against 67, 8 KiB (W=8, S=512, H=16, D=256) 73 against 66, 4 KiB at 1 GiB
// (W=8, S=4096, H=16, D=128) 77 against 75; but 3 KiB (D=96) 58 against 63,
// 6 KiB (H=24) 62 against 64, 14 KiB (W=8, S=4096, H=1, D=7168) 69 against 74
// and 16 KiB (W=16, S=2048, H=32, D=128 f32) 67 against 76.
constexpr int64_t kRowsMaxRun = 8 << 10;
// Default bytes per direct-mode piece: a tile's rows of one source larger than
// this are cut into ceil(bytes / kPieceBytes) pieces of equal token counts.
constexpr int64_t kPieceBytes = 128 << 10;
// Direct modes: with at least this many pieces (or row units) per compute unit,
// the persistent workgroups claim them dynamically, one workgroup per compute
// unit by default; with fewer, a static schedule with two per compute unit.
constexpr int64_t kDynPiecesPerCu = 8;

int lowbit_vec(uint64_t m) {
    if ((m & 15u) == 0) return 16;
    if ((m & 7u) == 0) return 8;
    if ((m & 3u) == 0) return 4;
    if ((m & 1u) == 0) return 2;
    return 1;
}

// Resolved tiling of one pipelined combine.
struct Plan {
    int64_t BS, TH, TD;
    int nbs, nhb, ndb, R;
    int MH, nmhb;           // head blocks moved together, merged head blocks
    int protocol;
    int64_t regionA, regionB;
    int64_t ring_bytes;     // staging ring bytes per slice
    int csplit, wg_per_cu, lookahead;
    int stream_batch;       // 0 = derive from the L2 budget
    int agent_sync;
    int direct;             // 1: direct push (no staging), 0: staged through the ring
    int rows;               // 1 (with direct): row units -- whole rows of out_j per unit
    int KU, upb;            // row units: tokens per unit, units per full S-block
    int PR, nsub;           // direct pieces: tokens per piece, pieces per tile and source
    int inverse;            // 1: the dispatch (the combine's inverse map)
    int bulk;               // 1: two-phase staging layout with fine-grained signals
    int pull;               // 1 (with bulk): staging in the sender's slice, pulled by the receiver
    int64_t piece_bytes, unit_bytes, tile_bytes;
};

int make_plan(int W, int64_t S, int64_t H, int64_t D, int e, const ra2a_opts_t* o, Plan* p) {
    ra2a_opts_t z;
    std::memset(&z, 0, sizeof z);
    z.straggler_rank = -1;
    if (!o) o = &z;
    if (o->reserved[0]) return fail(RA2A_EINVAL, "ra2a_opts_t.reserved must be zero");
    if (o->direction != RA2A_DIR_COMBINE && o->direction != RA2A_DIR_DISPATCH)
        return fail(RA2A_EINVAL, "direction must be RA2A_DIR_COMBINE or RA2A_DIR_DISPATCH");
    if (o->direction == RA2A_DIR_DISPATCH && (o->mode == RA2A_MODE_STAGED || o->mode == RA2A_MODE_BULK ||
                                              o->mode == RA2A_MODE_PULL))
        return fail(RA2A_EINVAL, "the dispatch runs in direct mode only");
    if (o->separate_reset != 0 && o->separate_reset != 1)
        return fail(RA2A_EINVAL, "separate_reset must be 0 or 1");
    if (o->mode != 0 && o->mode != RA2A_MODE_DIRECT && o->mode != RA2A_MODE_STAGED &&
        o->mode != RA2A_MODE_BULK && o->mode != RA2A_MODE_PULL && o->mode != RA2A_MODE_ROWS)
        return fail(RA2A_EINVAL, "mode must be 0, RA2A_MODE_ROWS, _DIRECT, _STAGED, _BULK or _PULL");
    if (o->mode == RA2A_MODE_ROWS && o->straggler_rank >= 0 && o->straggler_delay > 0)
        return fail(RA2A_EINVAL, "a straggler source needs per-source pieces: every row unit "
                                 "carries all sources (use RA2A_MODE_DIRECT)");
    if (o->unit_rows < 0) return fail(RA2A_EINVAL, "unit_rows must be >= 0");
    p->BS = o->tile_s > 0 ? o->tile_s : std::min<int64_t>(S, 64);
    p->TH = o->tile_h > 0 ? o->tile_h : 1;
    p->TD = o->tile_d > 0 ? o->tile_d : D;
    if (o->tile_s < 0 || o->tile_h < 0 || o->tile_d < 0)
        return fail(RA2A_EINVAL, "negative tile size");
    p->BS = std::min(p->BS, std::max<int64_t>(S, 1));
    p->TH = std::min(p->TH, H);
    p->TD = std::min(p->TD, D);
    if (o->protocol != 0 && o->protocol != RA2A_PROTO_ADD && o->protocol != RA2A_PROTO_SET)
        return fail(RA2A_EINVAL, "protocol must be 0, RA2A_PROTO_ADD or RA2A_PROTO_SET");
    p->inverse = o->direction == RA2A_DIR_DISPATCH ? 1 : 0;
    // the pull mode is the bulk mode's protocol with the staging on the sender's side
    p->pull = o->mode == RA2A_MODE_PULL ? 1 : 0;
    p->bulk = (o->mode == RA2A_MODE_BULK || p->pull) ? 1 : 0;
    // the dispatch fills each output tile from one source, and the bulk mode
    // signals each (S-block, sender): one signal per (tile, source), set to 1
    // (the SET layout)
    p->protocol = (o->protocol == RA2A_PROTO_SET || p->inverse || p->bulk) ? RA2A_SIG_SET
                                                                          : RA2A_SIG_ADD;
    p->nbs = (int)cdiv(S, p->BS);
    p->nhb = (int)cdiv(H, p->TH);
    p->ndb = (int)cdiv(D, p->TD);
    if (o->ring < 0) return fail(RA2A_EINVAL, "ring depth must be >= 0");
    int R = o->ring > 0 ? o->ring : 8;
    p->R = std::max(1, std::min(R, std::max(p->nbs, 1)));
    if (o->head_merge < 0) return fail(RA2A_EINVAL, "head_merge must be >= 0");
    if (o->head_merge > 0) {
        p->MH = std::min(o->head_merge, p->nhb);
    } else if (p->TD == D) {
        // adjacent head blocks are contiguous: merge up to ~4 KiB runs, but keep at
        // least kMinPieces pieces.  The direct modes need one for each of the (about
        // 512) persistent workgroups, since pieces above kPieceBytes move in parts
        // (measured on the W=8, S=512, H=16, D=128 bf16 shape, whole 4 KiB runs in
        // 256 KiB pieces of two parts against 2 KiB runs: the combine 48.2 against
        // 48.9 us, the dispatch, whose reads are the strided side, 51.1 against 53.0
        // us); the staged modes, whose pieces are not cut, two each.
        const bool direct_mode = !(o->mode == RA2A_MODE_STAGED || p->bulk);
        const int64_t kMinPieces = direct_mode ? 512 : 1024;
        int64_t mh = std::max<int64_t>(1, std::min<int64_t>(p->nhb, 4096 / std::max<int64_t>(1, p->TH * D * e)));
        const int64_t per_mh = (int64_t)W * p->nbs * W;  // pieces per merged head block
        while (mh > 1 && per_mh * cdiv(p->nhb, mh) < kMinPieces) mh /= 2;
        p->MH = (int)mh;
    } else {
        p->MH = 1;
    }
    p->nmhb = (p->nhb + p->MH - 1) / p->MH;
    const int64_t perW = p->protocol == RA2A_SIG_SET ? W : 1;
    p->regionA = (int64_t)p->nbs * p->nhb * p->ndb * perW;
    p->regionB = (int64_t)p->R * p->nmhb * p->ndb * perW;
    p->ring_bytes = (int64_t)p->R * p->BS * H * W * D * e;
    p->piece_bytes = p->BS * std::min<int64_t>((int64_t)p->MH * p->TH, H) * p->TD * e;
    p->tile_bytes = p->piece_bytes * W;  // one S-block of one stream, all sources
    if (o->stream_batch < 0) return fail(RA2A_EINVAL, "stream_batch must be >= 0");
    p->stream_batch = o->stream_batch;
    p->agent_sync = o->agent_sync ? 1 : 0;
    p->direct = (o->mode == RA2A_MODE_STAGED || p->bulk) ? 0 : 1;
    // Row units when asked for, and by default (the combine and the dispatch)
    // when a source's run of a token row (H*D*e) is at most kRowsMaxRun, divides
    // or is a multiple of the 4 KiB round, and nothing asks for per-source pieces
    // (a delayed straggler source, head merging or piece sizes set by the
    // caller); otherwise per-source pieces.
    const bool pieces_asked = (o->straggler_rank >= 0 && o->straggler_delay > 0) ||
                              o->head_merge > 0 || o->piece_rows > 0;
    const int64_t run = H * D * e;
    const bool rows_run = run <= kRowsMaxRun && run > 0 &&
                          (run % kRowWholeRun == 0 || kRowWholeRun % run == 0);
    p->rows = (o->mode == RA2A_MODE_ROWS || (o->mode == 0 && !pieces_asked && rows_run)) ? 1 : 0;
    p->unit_bytes = p->piece_bytes * (p->protocol == RA2A_SIG_SET ? 1 : W);
    if (o->consumer_split < 0 || o->wg_per_cu < 0 || o->lookahead < -1)
        return fail(RA2A_EINVAL, "negative option");
    // the kernels split a unit's vectors with 32-bit products part * (nvec mod cs)
    if (o->consumer_split > 4096) return fail(RA2A_EINVAL, "consumer_split above 4096");
    p->csplit = o->consumer_split > 0
                    ? o->consumer_split
                    : (int)std::max<int64_t>(1, std::min<int64_t>(64, p->unit_bytes / (128 << 10)));
    if (p->direct) {
        // no staging: no ring, no hand-back counters, no consumer work items
        p->R = std::max(p->nbs, 1);
        p->regionB = 0;
        p->ring_bytes = 0;
        p->csplit = 1;
    }
    // Tokens per piece.  In the staged modes a piece is a whole tile's rows of one
    // source.  In direct mode the rows of a tile may be cut into nsub parts, each
    // a piece of its own (about kPieceBytes by default), whose arrivals the tile
    // counts in region B (one counter per moved tile, per source under SET).
    p->PR = (int)p->BS;
    p->nsub = 1;
    if (o->piece_rows < 0) return fail(RA2A_EINVAL, "piece_rows must be >= 0");
    if (p->direct && !p->rows) {
        int64_t pr = p->BS;
        if (o->piece_rows > 0) {
            pr = std::min<int64_t>(o->piece_rows, p->BS);
        } else if (p->piece_bytes > kPieceBytes) {
            const int64_t parts = cdiv(p->piece_bytes, kPieceBytes);
            pr = cdiv(p->BS, parts);
        }
        p->PR = (int)pr;
        p->nsub = (int)cdiv(p->BS, pr);
        if (p->nsub > 1) p->regionB = (int64_t)p->nbs * p->nmhb * p->ndb * perW;
    }
    p->KU = 1;
    p->upb = 1;
    if (p->rows) {
        // tokens per row unit (default: about kRowUnitBytes of output, at least one
        // token, at most the S-block); region B holds one arrival counter per S-block
        const int64_t row_bytes = (int64_t)W * H * D * e;
        int64_t ku = o->unit_rows > 0 ? o->unit_rows : std::max<int64_t>(1, kRowUnitBytes / row_bytes);
        ku = std::min(ku, p->BS);
        if (o->unit_rows == 0 && H * D * e >= kRowWholeRun) {
            // runs of whole rounds: twice the bytes per unit while every compute
            // unit still gets one
            const int64_t ku2 = std::min<int64_t>(std::max<int64_t>(1, 2 * kRowUnitBytes / row_bytes), p->BS);
            const int64_t units2 = ((int64_t)(p->nbs - 1) * cdiv(p->BS, ku2) +
                                    cdiv(S - (int64_t)(p->nbs - 1) * p->BS, ku2)) * W;
            if (units2 >= kRowUnitsMin) ku = ku2;
        }
        p->KU = (int)ku;
        p->upb = (int)cdiv(p->BS, ku);
        p->regionB = p->nbs;
        p->unit_bytes = ku * row_bytes;
    }
    if (p->bulk) {
        // every sender's whole segment has a place: no ring reuse, no hand-back
        p->R = std::max(p->nbs, 1);
        p->regionB = 0;
        p->ring_bytes = (int64_t)W * S * H * D * e;
    }
    p->wg_per_cu = o->wg_per_cu;  // 0: resolved with the schedule at launch (prepare_pipelined)
    p->lookahead = o->lookahead;
    // the kernels index tiles, pieces and work items with 32-bit arithmetic
    const double tasks = (double)W * p->nbs * p->nhb * p->ndb * ((double)W + p->csplit * W);
    if (tasks >= 2147483647.0 - 65536.0) return fail(RA2A_EINVAL, "too many tiles");
    // per-launch index arithmetic uses 32-bit vector counts inside one unit
    if (p->unit_bytes >= (int64_t(1) << 31) - 65536) return fail(RA2A_EINVAL, "tile too large");
    // the direct modes store through a buffer descriptor per piece / unit, whose
    // range (at most one S-block of out_j rows) must stay below 2^32 bytes
    if (p->direct && (double)p->BS * W * H * D * e >= 4294967296.0 - 65536.0)
        return fail(RA2A_EINVAL, "an S-block of output rows (tile_s * W*H*D*e) reaches 4 GiB");
    // consumers address the staging ring with 32-bit buffer offsets
    if (p->ring_bytes >= (int64_t(1) << 32) && !(p->bulk && p->agent_sync))
        return fail(RA2A_EINVAL, "staging above 4 GiB per slice (the bulk mode allows it with "
                                 "agent_sync)");
    return RA2A_OK;
}

struct Checked {
    ra2a_heap* h;
    int e;
    int64_t n_bytes;  // per-slice bytes of in and of out
    size_t in_off, out_off, sig_off;
};

// Common validation of the combine's pointers and sizes.
int check_combine(const void* in, const void* out, const void* signals, int W, int64_t S,
                  int64_t H, int64_t D, int dtype, int64_t sig_slots, Checked* c) {
    c->e = elem_bytes(dtype);
    if (!c->e) return fail(RA2A_EINVAL, "unknown dtype %d", dtype);
    if (W < 1) return fail(RA2A_EINVAL, "W must be >= 1");
    if (S < 0 || H < 0 || D < 0) return fail(RA2A_EINVAL, "negative dimension");
    if (!in || !out) return fail(RA2A_EINVAL, "in and out must be non-NULL");
    c->h = find_heap(in);
    if (!c->h) return fail(RA2A_EINVAL, "in is not inside a symmetric heap");
    if (c->h->world != W)
        return fail(RA2A_EINVAL, "W=%d but the heap has %d slices", W, c->h->world);
    if (!in_heap(c->h, out)) return fail(RA2A_EINVAL, "out is not inside the heap of in");
    const double nb = (double)S * (double)W * (double)H * (double)D * (double)c->e;
    if (nb > 9.0e18) return fail(RA2A_EINVAL, "size overflow");
    c->n_bytes = S * (int64_t)W * H * D * c->e;
    c->in_off = sym_offset(c->h, in);
    c->out_off = sym_offset(c->h, out);
    if (c->in_off + (size_t)c->n_bytes > c->h->stride)
        return fail(RA2A_EINVAL, "in crosses the end of its slice");
    if (c->out_off + (size_t)c->n_bytes > c->h->stride)
        return fail(RA2A_EINVAL, "out crosses the end of its slice");
    if (c->n_bytes > 0 && c->in_off < c->out_off + (size_t)c->n_bytes &&
        c->out_off < c->in_off + (size_t)c->n_bytes)
        return fail(RA2A_EINVAL, "in and out overlap");
    if (sig_slots > 0) {
        if (!signals) return fail(RA2A_EINVAL, "signals must be non-NULL");
        if (!in_heap(c->h, signals)) return fail(RA2A_EINVAL, "signals not inside the heap of in");
        c->sig_off = sym_offset(c->h, signals);
        if (c->sig_off % 8) return fail(RA2A_EINVAL, "signals must be 8-byte aligned");
        const size_t sb = (size_t)sig_slots * RA2A_SIG_STRIDE_BYTES;
        if (c->sig_off + sb > c->h->stride)
            return fail(RA2A_EINVAL, "signals (%lld slots) cross the end of the slice",
                        (long long)sig_slots);
        if (c->n_bytes > 0 &&
            ((c->sig_off < c->in_off + (size_t)c->n_bytes && c->in_off < c->sig_off + sb) ||
             (c->sig_off < c->out_off + (size_t)c->n_bytes && c->out_off < c->sig_off + sb)))
            return fail(RA2A_EINVAL, "signals overlap in or out");
    }
    return RA2A_OK;
}

// Bump allocation under the heap's lock.
int heap_alloc(ra2a_heap* h, size_t bytes, size_t align, size_t* off) {
    // default: 4 KiB for buffers of 4 KiB or more (runs of 4 KiB, a round of
    // 256 lanes x 16 B, then keep to 4 KiB pages), 256 B below
    if (align == 0) align = bytes >= 4096 ? 4096 : 256;
    if (align & (align - 1)) return fail(RA2A_EINVAL, "align must be a power of two");
    const size_t start = (h->bump + align - 1) & ~(align - 1);
    if (start > h->stride || bytes > h->stride - start)
        return fail(RA2A_ENOMEM, "symmetric heap slice exhausted: need %zu bytes at offset %zu of %zu",
                    bytes, start, h->stride);
    h->bump = start + bytes;
    *off = start;
    return RA2A_OK;
}

// Staging area of at least `bytes` per slice, cached per heap.
int staging(ra2a_heap* h, bool full, size_t bytes, size_t* off) {
    if (g_no_alloc) return no_alloc_refused("staging");
    std::lock_guard<std::mutex> g(h->mu);
    size_t& co = full ? h->full_off : h->ring_off;
    size_t& cb = full ? h->full_bytes : h->ring_bytes;
    if (cb >= bytes && cb > 0) {
        *off = co;
        return RA2A_OK;
    }
    size_t o = 0;
    int rc = heap_alloc(h, std::max<size_t>(bytes, 256), 0, &o);
    if (rc) return fail(RA2A_ENOMEM, "staging of %zu bytes per slice does not fit the heap: %s",
                        bytes, g_err.c_str());
    co = o;
    cb = std::max<size_t>(bytes, 256);
    *off = o;
    return RA2A_OK;
}

int device_cus(int* n) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    e = hipDeviceGetAttribute(n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute(CU count)");
    return RA2A_OK;
}

int gcd_int(int a, int b) {
    while (b) {
        int t = a % b;
        a = b;
        b = t;
    }
    return a;
}

// Kernel arguments and launch shape of one pipelined combine (everything but the
// device pointers, error word and clock), shared by the launch and the host
// emulator.  Offsets are symmetric byte offsets inside a slice.
int prepare_pipelined(int W, int64_t S, int64_t H, int64_t D, int e0, const Plan& pl,
                      const ra2a_opts_t* opts, int64_t stride, size_t in_off, size_t out_off,
                      size_t stg_off, size_t sig_off, int ncu, int blocks_per_cu, int nxcd,
                      ra2a::PipeArgs* a, int* V, int* grid) {
    *a = ra2a::PipeArgs{};
    a->stride = stride;
    a->in_off = (int64_t)in_off;
    a->out_off = (int64_t)out_off;
    a->stg_off = (int64_t)stg_off;
    a->sig_off = (int64_t)sig_off;
    a->S = S;
    a->H = H;
    a->D = D;
    a->BS = pl.BS;
    a->TH = pl.TH;
    a->TD = pl.TD;
    a->W = W;
    a->e = e0;
    a->nbs = pl.nbs;
    a->nhb = pl.nhb;
    a->ndb = pl.ndb;
    a->MH = pl.MH;
    a->nmhb = pl.nmhb;
    a->R = pl.R;
    a->protocol = pl.protocol;
    const int nstreams = W * pl.nmhb * pl.ndb;
    // one stream group (and work queue) per XCD
    a->NG = std::max(1, std::min(nxcd, ra2a::kNumXcd));
    a->nstreams = nstreams;
    // XCD-local sync needs one group per XCD (XCC_ID mod NG must identify the XCD)
    // Direct mode publishes every tile device-wide: a tile's W pieces come from
    // workgroups on any XCD, and its consumer may run on any other.
    a->sync = (pl.agent_sync || pl.direct || nxcd > ra2a::kNumXcd) ? ra2a::kSyncAgent
                                                                   : ra2a::kSyncXcd;
    {
        const int ns_max = (nstreams + a->NG - 1) / a->NG;
        int kb = pl.stream_batch;
        if (kb <= 0) {
            const int64_t budget = int64_t(2) << 20;  // staging bytes per XCD kept in its L2
            kb = (int)std::max<int64_t>(1, budget / std::max<int64_t>(1, (int64_t)pl.R * pl.tile_bytes));
        }
        a->KB = std::max(1, std::min(kb, ns_max));
    }
    a->csplit = pl.csplit;
    a->lookahead = pl.lookahead;
    a->regionA = pl.regionA;
    a->regionB = pl.regionB;
    a->ring_bytes = pl.ring_bytes;
    a->direct = pl.direct;
    a->rows = pl.rows;
    a->KU = pl.KU;
    a->upb = pl.upb;
    // Row units: four rounds in flight per lane when each source's range in a
    // unit is at least 64 KiB, else eight (gfx950, bf16: W=8, S=512, H=16,
    // D=128, 64 KiB ranges, 46.3 against 46.9 us; D=256 91.2 against 93.5; W=16,
    // S=256, H=16, D=128, 32 KiB ranges, 92.4 against 90.2).
    a->ru = pl.rows && (int64_t)pl.KU * H * D * e0 >= (64 << 10) ? 4 : 8;
    a->PR = pl.PR;
    a->nsub = pl.nsub;
    a->inverse = pl.inverse;
    a->bulk = pl.bulk;
    a->pull = pl.pull;
    a->straggler = opts ? opts->straggler_rank : -1;
    a->delay = opts ? opts->straggler_delay : 0;
    a->seed = opts ? opts->straggler_seed : 0;
    a->units_per_dest = pl.regionA;
    // vector width: every offset, stride and run is a multiple of it
    const uint64_t m = (uint64_t)(D * e0) | (uint64_t)(pl.TD * e0) | in_off | out_off | stg_off;
    *V = lowbit_vec(m);
    // Schedule of the direct modes: for pieces, dynamic claims when they are many
    // per compute unit, else static; workgroups per compute unit as asked, else
    // one (dynamic, and row units) or two (static pieces; on the W=8, S=512, H=16,
    // D=128 bf16 shape the dispatch measured 51.1 us with two against 53.1 with
    // one).  The staged modes keep two by default.
    int64_t work = 0;
    if (pl.rows) {
        a->nunits = ra2a::total_row_units(*a);
        if (a->nunits >= (int64_t(1) << 31) - 65536) return fail(RA2A_EINVAL, "too many row units");
        work = a->nunits;
    } else if (pl.direct) {
        work = ra2a::total_pieces(*a);
    }
    // Row units keep the static schedule with one workgroup per compute unit:
    // on gfx950 fewer copies in flight fill HBM better here (W=8, S=4096, H=16,
    // D=128 bf16, 256 KiB units: 350 us static against 378 claimed; W=8, S=512:
    // 47.5 against 48.0 us with two per compute unit).
    a->dyn = pl.direct && !pl.rows && work >= kDynPiecesPerCu * (int64_t)ncu ? 1 : 0;
    int wpc = pl.wg_per_cu;
    if (wpc <= 0) wpc = (pl.rows || (pl.direct && a->dyn)) ? 1 : 2;
    const int per_cu = std::max(1, std::min(blocks_per_cu, wpc));
    *grid = per_cu * ncu;
    if (pl.direct) *grid = (int)std::min<int64_t>(*grid, work);  // no workgroup without work
    // the claim counter: the spare queue word (slice 0), zeroed with the signals
    a->claim_off = (int64_t)sig_off + (pl.regionA + pl.regionB + ra2a::kQueueSlots - 1) *
                                          RA2A_SIG_STRIDE_BYTES;
    if (*grid < 1) return fail(RA2A_EUNSUPPORTED, "no compute units");
    return RA2A_OK;
}

// Number of XCDs of the current device (the largest XCC_ID a probe launch of
// 4096 workgroups observed, plus one), measured once per device.
std::mutex& g_xcd_mu = *new std::mutex;
int g_xcd_n[64];  // per device: measured XCD count, 0 = not measured yet

int xcd_count(int* nxcd) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= 64) {
        *nxcd = 1;
        return RA2A_OK;
    }
    std::lock_guard<std::mutex> g(g_xcd_mu);
    int* cached_n = g_xcd_n;
    if (!cached_n[dev]) {
        if (g_no_alloc) return no_alloc_refused("the XCD probe");
        const int n = 4096;
        uint32_t* d = nullptr;
        e = hipMalloc(&d, n * sizeof(uint32_t));
        if (e != hipSuccess) return hip_fail(e, "probe allocation");
        e = ra2a::launch_xcc_probe(d, n, nullptr);
        if (e == hipSuccess) e = hipDeviceSynchronize();
        std::vector<uint32_t> h(n, 0);
        if (e == hipSuccess) e = hipMemcpy(h.data(), d, n * sizeof(uint32_t), hipMemcpyDeviceToHost);
        (void)hipFree(d);
        if (e != hipSuccess) return hip_fail(e, "XCD probe");
        uint32_t mx = 0;
        for (uint32_t v : h) mx = std::max(mx, v);
        cached_n[dev] = (int)mx + 1;
    }
    *nxcd = cached_n[dev];
    return RA2A_OK;
}

// The current device's XCD count if an earlier call measured it (no probe).
bool xcd_count_known(int* nxcd) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return false;
    std::lock_guard<std::mutex> g(g_xcd_mu);
    if (!g_xcd_n[dev]) return false;
    *nxcd = g_xcd_n[dev];
    return true;
}

// Tag of one in-launch reset: a process-wide counter starting at a random
// value, never 0, so a reset flag left by any earlier launch never matches.
uint64_t next_reset_tag() {
    static std::atomic<uint64_t> ctr{[] {
        std::random_device rd;
        const uint64_t t = (uint64_t)std::chrono::steady_clock::now().time_since_epoch().count();
        return ((uint64_t)rd() << 32) ^ (uint64_t)rd() ^ (t * 0x9E3779B97F4A7C15ull);
    }()};
    uint64_t t;
    do t = ctr.fetch_add(1, std::memory_order_relaxed);
    while (t == 0);
    return t;
}

int combine_pipelined(const void* in, void* out, uint64_t* signals, int W, int64_t S, int64_t H,
                      int64_t D, int dtype, const ra2a_opts_t* opts, void* stream) {
    const int e0 = elem_bytes(dtype);
    if (!e0) return fail(RA2A_EINVAL, "unknown dtype %d", dtype);
    if (W < 1) return fail(RA2A_EINVAL, "W must be >= 1");
    if (S < 0 || H < 0 || D < 0) return fail(RA2A_EINVAL, "negative dimension");
    Plan pl{};
    const bool empty = S == 0 || H == 0 || D == 0;
    if (!empty) {
        int rc = make_plan(W, S, H, D, e0, opts, &pl);
        if (rc) return rc;
    }
    Checked c{};
    int rc = check_combine(in, out, signals, W, S, H, D, dtype,
                           empty ? 0 : pl.regionA + pl.regionB + ra2a::kQueueSlots + ra2a::kResetFlags,
                           &c);
    if (rc) return rc;
    if (empty) return ok();
    if (opts && (opts->straggler_rank < -1 || opts->straggler_rank >= W))
        return fail(RA2A_EINVAL, "straggler_rank out of range");
    size_t stg = 0;
    if (!pl.direct) {
        rc = staging(c.h, false, (size_t)pl.ring_bytes, &stg);
        if (rc) return rc;
    }
    rc = ensure_err(c.h);
    if (rc) return rc;

    int ncu = 0;
    rc = device_cus(&ncu);
    if (rc) return rc;
    int nxcd = 1;
    rc = xcd_count(&nxcd);
    if (rc) return rc;
    const uint64_t m = (uint64_t)(D * e0) | (uint64_t)(pl.TD * e0) | c.in_off | c.out_off | stg;
    int occ = 0;
    hipError_t he = ra2a::pipelined_blocks_per_cu(
        lowbit_vec(m), (pl.agent_sync || pl.direct) ? ra2a::kSyncAgent : ra2a::kSyncXcd, pl.direct,
        &occ);
    if (he != hipSuccess) return hip_fail(he, "occupancy query");
    ra2a::PipeArgs a{};
    int V = 16, grid = 0;
    rc = prepare_pipelined(W, S, H, D, e0, pl, opts, (int64_t)c.h->stride, c.in_off, c.out_off,
                           stg, c.sig_off, ncu, occ, nxcd, &a, &V, &grid);
    if (rc) return rc;
    a.base = c.h->base;
    a.err = c.h->err;
    a.stamps = opts ? opts->timestamps : nullptr;
    a.timeout = timeout_ticks(c.h);
    a.piece_grid = grid;

    hipStream_t st = static_cast<hipStream_t>(stream);
    const bool skip = opts && opts->skip_reset;
    const int64_t reset_slots = pl.regionA + pl.regionB + ra2a::kQueueSlots;
    const int64_t nstamps = a.stamps ? (int64_t)W * pl.regionA : 0;
    // In-launch reset: direct mode, unless asked for a separate launch.  The
    // zeroing workgroups take the launch's lowest block ids, so they are
    // dispatched before any workgroup that waits for them, whatever else occupies
    // the device.  Not under stream capture: a replayed launch would carry the tag
    // it was captured with, the reset flags would already hold it, and producers
    // could signal before the zeroing.
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    he = hipStreamIsCapturing(st, &cap);
    if (he != hipSuccess) return hip_fail(he, "hipStreamIsCapturing");
    const bool in_launch = pl.direct && !(opts && opts->separate_reset) &&
                           (!skip || nstamps > 0) && cap == hipStreamCaptureStatusNone;
    if (in_launch) {
        // at most about 16 slots per thread and zeroing workgroup, a multiple of the
        // XCD count of them (one or more on every XCD), at most kResetFlags.  On the
        // W=8, S=512, H=16, D=128 bf16 shape the dispatch (three zeroing workgroups
        // by the first rule alone) measured 48.4-49.5 us against 47.5 with eight,
        // 47.7 with sixteen and 48.4 with 32; the combine (one) 47.0 against 46.8.
        const int64_t work = (skip ? 0 : reset_slots * W) + nstamps;  // words to zero
        const int64_t nz_work = std::max<int64_t>(1, (work + 16 * ra2a::kThreads - 1) / (16 * ra2a::kThreads));
        const int64_t per_xcd = std::max(1, nxcd);
        const int64_t nz = std::min<int64_t>(ra2a::kResetFlags, (nz_work + per_xcd - 1) / per_xcd * per_xcd);
        a.reset_tag = next_reset_tag();
        a.reset_nz = (int)nz;
        a.reset_slots = skip ? 0 : reset_slots;  // skip_reset: the caller zeroed the signals
        a.reset_chunk = (a.reset_slots + nz - 1) / nz;
        a.stamp_chunk = (nstamps + nz - 1) / nz;
        a.flag_off = (int64_t)c.sig_off + reset_slots * RA2A_SIG_STRIDE_BYTES;
        grid += (int)nz;
    } else {
        if (!skip) {
            he = ra2a::launch_signal_reset(c.h->base, (int64_t)c.h->stride, W, (int64_t)c.sig_off,
                                           reset_slots, st);
            if (he != hipSuccess) return hip_fail(he, "signal reset launch");
        }
        he = ra2a::launch_zero_u64(a.stamps, nstamps, st);
        if (he != hipSuccess) return hip_fail(he, "timestamp reset");
    }
    he = ra2a::launch_pipelined(a, V, grid, st);
    if (he != hipSuccess) return hip_fail(he, "pipelined combine launch");
    return ok();
}

}  // namespace

// ===========================================================================
// heap

RA2A_API int ra2a_symm_heap_create(int world, size_t slice_bytes, ra2a_heap_t** out) {
    if (!out) return fail(RA2A_EINVAL, "out must be non-NULL");
    *out = nullptr;
    if (world < 1 || world > 4096) return fail(RA2A_EINVAL, "world must be in [1, 4096]");
    if (slice_bytes == 0) return fail(RA2A_EINVAL, "slice_bytes must be > 0");
    const size_t stride = (slice_bytes + kSliceAlign - 1) / kSliceAlign * kSliceAlign;
    if (stride / kSliceAlign > (SIZE_MAX / kSliceAlign) / (size_t)world)
        return fail(RA2A_EINVAL, "heap size overflow");
    ra2a_heap* h = new (std::nothrow) ra2a_heap;
    if (!h) return fail(RA2A_ENOMEM, "host allocation failed");
    h->world = world;
    h->stride = stride;
    hipError_t e = hipGetDevice(&h->device);
    if (e != hipSuccess) {
        delete h;
        return hip_fail(e, "hipGetDevice");
    }
    void* p = nullptr;
    e = hipMalloc(&p, stride * (size_t)world);
    if (e != hipSuccess) {
        delete h;
        (void)hipGetLastError();
        return fail(e == hipErrorOutOfMemory ? RA2A_ENOMEM : RA2A_EHIP,
                    "hipMalloc of %zu bytes: %s", stride * (size_t)world, hipGetErrorString(e));
    }
    h->base = static_cast<uint8_t*>(p);
    {
        std::lock_guard<std::mutex> g(g_reg_mu);
        g_heaps.push_back(h);
    }
    *out = h;
    return ok();
}

RA2A_API int ra2a_symm_heap_attach(void* base, int world, size_t stride, ra2a_heap_t** out) {
    if (!out) return fail(RA2A_EINVAL, "out must be non-NULL");
    *out = nullptr;
    if (!base) return fail(RA2A_EINVAL, "base must be non-NULL");
    if (world < 1 || world > 4096) return fail(RA2A_EINVAL, "world must be in [1, 4096]");
    if (stride == 0 || stride % 256 || (uintptr_t)base % 256)
        return fail(RA2A_EINVAL, "base and stride must be non-zero multiples of 256");
    if (stride > SIZE_MAX / (size_t)world) return fail(RA2A_EINVAL, "heap size overflow");
    const uint8_t* b = static_cast<const uint8_t*>(base);
    {
        std::lock_guard<std::mutex> g(g_reg_mu);
        for (ra2a_heap* o : g_heaps)
            if (b < o->base + o->stride * (size_t)o->world && o->base < b + stride * (size_t)world)
                return fail(RA2A_EINVAL, "range overlaps a live heap");
    }
    ra2a_heap* h = new (std::nothrow) ra2a_heap;
    if (!h) return fail(RA2A_ENOMEM, "host allocation failed");
    h->world = world;
    h->stride = stride;
    h->base = static_cast<uint8_t*>(base);
    h->owned = false;
    {
        std::lock_guard<std::mutex> g(g_reg_mu);
        g_heaps.push_back(h);
    }
    *out = h;
    return ok();
}

RA2A_API int ra2a_symm_heap_destroy(ra2a_heap_t* h) {
    if (!h) return ok();
    {
        std::lock_guard<std::mutex> g(g_reg_mu);
        auto it = std::find(g_heaps.begin(), g_heaps.end(), h);
        if (it == g_heaps.end()) return fail(RA2A_EINVAL, "not a live heap");
        g_heaps.erase(it);
    }
    if (g_exiting.load()) {  // too late for HIP calls (see mark_exiting)
        delete h;
        return ok();
    }
    const bool touched = h->owned || h->err || h->bt_ws;
    hipError_t e = touched ? hipDeviceSynchronize() : hipSuccess;
    hipError_t e1 = h->owned ? hipFree(h->base) : hipSuccess;
    hipError_t e2 = h->err ? hipFree(h->err) : hipSuccess;
    hipError_t e3 = h->bt_ws ? hipFree(h->bt_ws) : hipSuccess;
    delete h;
    if (e3 != hipSuccess) return hip_fail(e3, "hipFree(B^T workspace)");
    if (e != hipSuccess) return hip_fail(e, "hipDeviceSynchronize");
    if (e1 != hipSuccess) return hip_fail(e1, "hipFree(heap)");
    if (e2 != hipSuccess) return hip_fail(e2, "hipFree(error word)");
    return ok();
}

RA2A_API int ra2a_symm_malloc(ra2a_heap_t* h, size_t bytes, size_t align, size_t* sym_offset_out) {
    if (!h || !sym_offset_out) return fail(RA2A_EINVAL, "heap and sym_offset must be non-NULL");
    std::lock_guard<std::mutex> g(h->mu);
    return heap_alloc(h, bytes, align, sym_offset_out);
}

RA2A_API int ra2a_symm_heap_info(const ra2a_heap_t* h, void** base, size_t* stride, int* world) {
    if (!h) return fail(RA2A_EINVAL, "heap must be non-NULL");
    if (base) *base = h->base;
    if (stride) *stride = h->stride;
    if (world) *world = h->world;
    return ok();
}

RA2A_API ra2a_heap_t* ra2a_symm_heap_find(const void* ptr) { return find_heap(ptr); }

RA2A_API void* ra2a_symm_at(const ra2a_heap_t* h, const void* ptr, int rank) {
    if (!h || !in_heap(h, ptr) || rank < 0 || rank >= h->world) return nullptr;
    return h->base + (size_t)rank * h->stride + sym_offset(h, ptr);
}

RA2A_API int ra2a_symm_heap_set_spin_timeout(ra2a_heap_t* h, uint64_t timeout_us) {
    if (!h) return fail(RA2A_EINVAL, "heap must be non-NULL");
    h->timeout_us = timeout_us;
    return ok();
}

// ===========================================================================
// primitives

namespace {

int check_remote(const ra2a_heap_t* h, const void* sym, size_t bytes, int rank, const char* what,
                 uint8_t** dst) {
    if (!h) return fail(RA2A_EINVAL, "heap must be non-NULL");
    if (!sym || !in_heap(h, sym)) return fail(RA2A_EINVAL, "%s is not inside the heap", what);
    if (rank < 0 || rank >= h->world)
        return fail(RA2A_EINVAL, "target rank %d outside [0, %d)", rank, h->world);
    const size_t off = sym_offset(h, sym);
    if (bytes > h->stride - off) return fail(RA2A_EINVAL, "%s range crosses the end of the slice", what);
    *dst = h->base + (size_t)rank * h->stride + off;
    return RA2A_OK;
}

int check_sig(const ra2a_heap_t* h, const uint64_t* sig, int rank, uint64_t** out) {
    uint8_t* p = nullptr;
    int rc = check_remote(h, sig, 8, rank, "signal", &p);
    if (rc) return rc;
    if ((uintptr_t)p % 8) return fail(RA2A_EINVAL, "signal must be 8-byte aligned");
    *out = reinterpret_cast<uint64_t*>(p);
    return RA2A_OK;
}

}  // namespace

RA2A_API int ra2a_put(const ra2a_heap_t* h, void* dst_sym, const void* src, size_t bytes,
                      int target_rank, void* stream) {
    uint8_t* dst = nullptr;
    int rc = check_remote(h, dst_sym, bytes, target_rank, "dst", &dst);
    if (rc) return rc;
    if (bytes && !src) return fail(RA2A_EINVAL, "src must be non-NULL");
    const uint8_t* s = static_cast<const uint8_t*>(src);
    if (bytes && s < dst + bytes && dst < s + bytes) return fail(RA2A_EINVAL, "src and dst overlap");
    hipError_t e = ra2a::launch_put(dst, s, (int64_t)bytes, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "put launch");
    return ok();
}

RA2A_API int ra2a_get(const ra2a_heap_t* h, void* dst, const void* src_sym, size_t bytes,
                      int source_rank, void* stream) {
    uint8_t* src = nullptr;
    int rc = check_remote(h, src_sym, bytes, source_rank, "src", &src);
    if (rc) return rc;
    if (bytes && !dst) return fail(RA2A_EINVAL, "dst must be non-NULL");
    uint8_t* d = static_cast<uint8_t*>(dst);
    if (bytes && d < src + bytes && src < d + bytes) return fail(RA2A_EINVAL, "src and dst overlap");
    hipError_t e = ra2a::launch_put(d, src, (int64_t)bytes, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "get launch");
    return ok();
}

RA2A_API int ra2a_put_with_signal(const ra2a_heap_t* h, void* dst_sym, const void* src, size_t bytes,
                                  uint64_t* sig_sym, uint64_t value, int sig_op, int target_rank,
                                  void* stream) {
    uint8_t* dst = nullptr;
    int rc = check_remote(h, dst_sym, bytes, target_rank, "dst", &dst);
    if (rc) return rc;
    uint64_t* sig = nullptr;
    rc = check_sig(h, sig_sym, target_rank, &sig);
    if (rc) return rc;
    if (sig_op != RA2A_SIG_SET && sig_op != RA2A_SIG_ADD)
        return fail(RA2A_EINVAL, "sig_op must be RA2A_SIG_SET or RA2A_SIG_ADD");
    if (bytes && !src) return fail(RA2A_EINVAL, "src must be non-NULL");
    const uint8_t* s = static_cast<const uint8_t*>(src);
    if (bytes && s < dst + bytes && dst < s + bytes) return fail(RA2A_EINVAL, "src and dst overlap");
    const uint8_t* sg = reinterpret_cast<const uint8_t*>(sig);
    if (bytes && sg < dst + bytes && dst < sg + 8) return fail(RA2A_EINVAL, "signal inside dst range");
    hipError_t e = ra2a::launch_put_with_signal(dst, s, (int64_t)bytes, sig, value, sig_op,
                                                static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "put_with_signal launch");
    return ok();
}

RA2A_API int ra2a_signal_op(const ra2a_heap_t* h, uint64_t* sig_sym, uint64_t value, int sig_op,
                            int target_rank, void* stream) {
    uint64_t* sig = nullptr;
    int rc = check_sig(h, sig_sym, target_rank, &sig);
    if (rc) return rc;
    if (sig_op != RA2A_SIG_SET && sig_op != RA2A_SIG_ADD)
        return fail(RA2A_EINVAL, "sig_op must be RA2A_SIG_SET or RA2A_SIG_ADD");
    hipError_t e = ra2a::launch_signal_op(sig, value, sig_op, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "signal launch");
    return ok();
}

RA2A_API int ra2a_wait_signal(const ra2a_heap_t* h, const uint64_t* sig, uint64_t cmp_value,
                              int cmp_op, void* stream) {
    if (!h) return fail(RA2A_EINVAL, "heap must be non-NULL");
    if (!sig || !in_heap(h, sig)) return fail(RA2A_EINVAL, "signal is not inside the heap");
    if ((uintptr_t)sig % 8) return fail(RA2A_EINVAL, "signal must be 8-byte aligned");
    if (sym_offset(h, sig) + 8 > h->stride) return fail(RA2A_EINVAL, "signal crosses the slice end");
    if (cmp_op < RA2A_CMP_EQ || cmp_op > RA2A_CMP_LE) return fail(RA2A_EINVAL, "bad cmp_op");
    ra2a_heap* hh = const_cast<ra2a_heap*>(h);
    int rc = ensure_err(hh);
    if (rc) return rc;
    hipError_t e = ra2a::launch_wait(sig, cmp_op, cmp_value, timeout_ticks(h), h->err,
                                     static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "wait launch");
    return ok();
}

RA2A_API int ra2a_signal_reset(const ra2a_heap_t* h, uint64_t* sig_sym, int64_t n_slots,
                               void* stream) {
    if (!h) return fail(RA2A_EINVAL, "heap must be non-NULL");
    if (n_slots < 0) return fail(RA2A_EINVAL, "n_slots must be >= 0");
    if (n_slots == 0) return ok();
    if (!sig_sym || !in_heap(h, sig_sym)) return fail(RA2A_EINVAL, "signals not inside the heap");
    const size_t off = sym_offset(h, sig_sym);
    if (off % 8) return fail(RA2A_EINVAL, "signals must be 8-byte aligned");
    if ((size_t)(n_slots - 1) > (h->stride - off - 8) / RA2A_SIG_STRIDE_BYTES || off + 8 > h->stride)
        return fail(RA2A_EINVAL, "signal slots cross the end of the slice");
    hipError_t e = ra2a::launch_signal_reset(h->base, (int64_t)h->stride, h->world, (int64_t)off,
                                             n_slots, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "signal reset launch");
    return ok();
}

// ===========================================================================
// combine

RA2A_API int ra2a_rev_all2all_signal_slots(int W, int64_t S, int64_t H, int64_t D, int dtype,
                                           const ra2a_opts_t* opts, int64_t* tile_slots,
                                           int64_t* credit_slots, int64_t* queue_slots) {
    const int e = elem_bytes(dtype);
    if (!e) return fail(RA2A_EINVAL, "unknown dtype %d", dtype);
    if (W < 1 || S < 0 || H < 0 || D < 0) return fail(RA2A_EINVAL, "bad dimensions");
    int64_t a = 0, b = 0;
    if (S > 0 && H > 0 && D > 0) {
        Plan p{};
        int rc = make_plan(W, S, H, D, e, opts, &p);
        if (rc) return rc;
        a = p.regionA;
        b = p.regionB;
    }
    if (tile_slots) *tile_slots = a;
    if (credit_slots) *credit_slots = b;
    if (queue_slots) *queue_slots = (a + b) > 0 ? ra2a::kQueueSlots + ra2a::kResetFlags : 0;
    return ok();
}

RA2A_API int ra2a_rev_all2all_plan(int W, int64_t S, int64_t H, int64_t D, int dtype,
                                   const ra2a_opts_t* opts, ra2a_plan_t* plan) {
    const int e = elem_bytes(dtype);
    if (!e) return fail(RA2A_EINVAL, "unknown dtype %d", dtype);
    if (!plan) return fail(RA2A_EINVAL, "plan must be non-NULL");
    if (W < 1 || S < 1 || H < 1 || D < 1) return fail(RA2A_EINVAL, "bad dimensions");
    Plan p{};
    int rc = make_plan(W, S, H, D, e, opts, &p);
    if (rc) return rc;
    std::memset(plan, 0, sizeof *plan);
    plan->mode = p.rows ? RA2A_MODE_ROWS
                 : p.direct ? RA2A_MODE_DIRECT
                 : p.pull   ? RA2A_MODE_PULL
                 : p.bulk   ? RA2A_MODE_BULK
                            : RA2A_MODE_STAGED;
    plan->protocol = p.protocol == RA2A_SIG_SET ? RA2A_PROTO_SET : RA2A_PROTO_ADD;
    plan->tile_s = p.BS;
    plan->tile_h = p.TH;
    plan->tile_d = p.TD;
    plan->head_merge = p.MH;
    plan->piece_rows = p.PR;
    plan->pieces_per_tile = p.nsub;
    plan->unit_rows = p.rows ? p.KU : 0;
    plan->tile_slots = p.regionA;
    plan->credit_slots = p.regionB;
    plan->queue_slots = ra2a::kQueueSlots + ra2a::kResetFlags;
    plan->workspace_bytes = (size_t)p.ring_bytes;
    if (p.direct) {
        ra2a::PipeArgs a{};
        int V = 16, grid = 0;
        rc = prepare_pipelined(W, S, H, D, e, p, opts, int64_t(1) << 40, 0, 0, 0, 0, 256, 8, 8, &a,
                               &V, &grid);
        if (rc) return rc;
        plan->work_items = p.rows ? a.nunits : ra2a::total_pieces(a);
    }
    return ok();
}

RA2A_API int ra2a_rev_all2all_workspace_bytes(int W, int64_t S, int64_t H, int64_t D, int dtype,
                                              const ra2a_opts_t* opts, int two_phase, size_t* bytes) {
    const int e = elem_bytes(dtype);
    if (!e) return fail(RA2A_EINVAL, "unknown dtype %d", dtype);
    if (W < 1 || S < 0 || H < 0 || D < 0 || !bytes) return fail(RA2A_EINVAL, "bad arguments");
    if (S == 0 || H == 0 || D == 0) {
        *bytes = 0;
        return ok();
    }
    if (two_phase) {
        *bytes = (size_t)(S * (int64_t)W * H * D * e);
        return ok();
    }
    Plan p{};
    int rc = make_plan(W, S, H, D, e, opts, &p);
    if (rc) return rc;
    *bytes = (size_t)p.ring_bytes;
    return ok();
}

RA2A_API int ra2a_rev_all2all(const void* in, void* out, uint64_t* signals, int W, int64_t S,
                              int64_t H, int64_t D, int dtype, void* stream) {
    return combine_pipelined(in, out, signals, W, S, H, D, dtype, nullptr, stream);
}

RA2A_API int ra2a_rev_all2all_ex(const void* in, void* out, uint64_t* signals, int W, int64_t S,
                                 int64_t H, int64_t D, int dtype, const ra2a_opts_t* opts,
                                 void* stream) {
    return combine_pipelined(in, out, signals, W, S, H, D, dtype, opts, stream);
}

RA2A_API int ra2a_all2all_dispatch(const void* in, void* out, uint64_t* signals, int W, int64_t S,
                                   int64_t H, int64_t D, int dtype, void* stream) {
    return ra2a_all2all_dispatch_ex(in, out, signals, W, S, H, D, dtype, nullptr, stream);
}

RA2A_API int ra2a_all2all_dispatch_ex(const void* in, void* out, uint64_t* signals, int W,
                                      int64_t S, int64_t H, int64_t D, int dtype,
                                      const ra2a_opts_t* opts, void* stream) {
    ra2a_opts_t o;
    if (opts) {
        o = *opts;
    } else {
        std::memset(&o, 0, sizeof o);
        o.straggler_rank = -1;
    }
    o.direction = RA2A_DIR_DISPATCH;
    return combine_pipelined(in, out, signals, W, S, H, D, dtype, &o, stream);
}

RA2A_API int ra2a_rev_all2all_two_phase(const void* in, void* out, uint64_t* signals, int W,
                                        int64_t S, int64_t H, int64_t D, int dtype, void* stream) {
    (void)signals;
    Checked c{};
    int rc = check_combine(in, out, nullptr, W, S, H, D, dtype, 0, &c);
    if (rc) return rc;
    if (c.n_bytes == 0) return ok();
    size_t stg = 0;
    rc = staging(c.h, true, (size_t)c.n_bytes, &stg);
    if (rc) return rc;
    ra2a::TwoPhaseArgs a{};
    a.base = c.h->base;
    a.stride = (int64_t)c.h->stride;
    a.in_off = (int64_t)c.in_off;
    a.out_off = (int64_t)c.out_off;
    a.stg_off = (int64_t)stg;
    a.S = S;
    a.H = H;
    a.D = D;
    a.W = W;
    a.e = c.e;
    const uint64_t m = (uint64_t)(H * D * c.e) | c.in_off | c.out_off | stg;
    const int V = lowbit_vec(m);
    if (c.n_bytes / V >= (int64_t(1) << 31))
        return fail(RA2A_EUNSUPPORTED, "two-phase combine: more than 2^31 vectors per slice");
    hipError_t e = ra2a::launch_two_phase(a, V, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "two-phase launch");
    return ok();
}

// ===========================================================================
// AllGather + GEMM

namespace {

// Plan of one AllGather+GEMM: everything but the device pointers.
int plan_ag_gemm(int W, int rank, int64_t m_local, int64_t K, int64_t N, int tile_rows, int nxcd,
                 bool agent_sync, ra2a::AgGemmArgs* a) {
    if (W < 1) return fail(RA2A_EINVAL, "W must be >= 1");
    if (rank < 0 || rank >= W) return fail(RA2A_EINVAL, "rank %d out of [0, %d)", rank, W);
    if (m_local < 1 || K < 1 || N < 1) return fail(RA2A_EINVAL, "m_local, K and N must be >= 1");
    if (K % 8 || N % 8) return fail(RA2A_EINVAL, "K and N must be multiples of 8 (16-byte rows)");
    if (tile_rows < 1) return fail(RA2A_EINVAL, "tile_rows must be >= 1");
    *a = ra2a::AgGemmArgs{};
    a->W = W;
    a->rank = rank;
    a->m_local = m_local;
    a->K = K;
    a->N = N;
    const int64_t tr = std::min<int64_t>(tile_rows, m_local);
    a->tile_rows = (int)tr;
    a->ntiles = (int)cdiv(m_local, tr);
    // AllGather parts of about 128 KiB, never straddling a tile
    const int64_t row_bytes = K * 2;
    const int64_t np0 = std::max<int64_t>(1, cdiv(tr * row_bytes, int64_t(128) << 10));
    a->rpp = (int)cdiv(tr, np0);
    a->np = (int)cdiv(tr, a->rpp);
    const int64_t rows_last = m_local - (int64_t)(a->ntiles - 1) * tr;
    a->np_last = (int)cdiv(rows_last, a->rpp);
    a->nmb = (int)cdiv(m_local, ra2a::kGemmBM);
    a->ncol = (int)cdiv(N, ra2a::kGemmBN);
    a->NG = std::max(1, std::min(nxcd, ra2a::kNumXcd));
    a->spg = (int)cdiv(W, a->NG);
    a->sync = (agent_sync || nxcd > ra2a::kNumXcd) ? ra2a::kSyncAgent : ra2a::kSyncXcd;
    a->ntasks_shard = ra2a::agg_tasks_per_shard(*a);
    if ((double)a->ntasks_shard * a->spg >= 2147483647.0 - 65536.0 ||
        (double)a->rpp * row_bytes >= 2147483647.0)
        return fail(RA2A_EINVAL, "AllGather+GEMM too large for 32-bit task indices");
    // a GEMM tile's operand rows are addressed with 32-bit buffer offsets
    if ((double)ra2a::kGemmBM * row_bytes >= 4294967295.0 - 65536.0)
        return fail(RA2A_EINVAL, "K too large for 32-bit operand offsets");
    return RA2A_OK;
}

}  // namespace

RA2A_API int ra2a_ag_gemm_signal_slots(int W, int64_t m_local, int tile_rows, int64_t* tile_slots,
                                       int64_t* count_slots, int64_t* queue_slots) {
    if (W < 1 || m_local < 1 || tile_rows < 1) return fail(RA2A_EINVAL, "bad arguments");
    const int64_t tr = std::min<int64_t>(tile_rows, m_local);
    const int64_t nt = (int64_t)W * cdiv(m_local, tr);
    if (tile_slots) *tile_slots = nt;
    if (count_slots) *count_slots = nt;
    if (queue_slots) *queue_slots = ra2a::kQueueSlots;
    return ok();
}

namespace {

// The allocation-free entry points keep their workspace and error word in one
// static device array per GPU (`scratch`): the first kScratchErrBytes hold the
// error word, the rest the B^T workspace of ra2a_ag_gemm_noalloc.  Host code
// never passes the array's name to a kernel or a copy (on the host it is only
// a stand-in): it uses the device address hipGetSymbolAddress gives for the
// current device, looked up once per device and kept in g_scratch.
constexpr size_t kScratchErrBytes = 256;
constexpr size_t kScratchBtBytes = size_t(64) << 20;
__device__ __align__(256) uint8_t scratch[kScratchErrBytes + kScratchBtBytes];

constexpr int kMaxDevices = 64;
std::mutex& g_scratch_mu = *new std::mutex;
uint8_t* g_scratch[kMaxDevices];  // per device: scratch's device address, or null

// The current device's scratch address (looked up on first use).
int scratch_address(uint8_t** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(RA2A_EUNSUPPORTED, "device index %d", dev);
    std::lock_guard<std::mutex> g(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        g_scratch[dev] = static_cast<uint8_t*>(p);
    }
    *out = g_scratch[dev];
    return RA2A_OK;
}

// Shared by ra2a_ag_gemm and ra2a_ag_gemm_noalloc.  `no_alloc`: B^T goes to the
// device's scratch array (at most kScratchBtBytes) and errors to its error word;
// the XCD count is used only if an earlier call measured it (else device-wide
// synchronisation, which needs no placement knowledge).
int ag_gemm_run(const void* a_shards, void* gathered, const void* b, void* c, uint64_t* signals,
                int W, int rank, int64_t m_local, int64_t K, int64_t N, int tile_rows, int flags,
                void* stream, bool no_alloc) {
    if (flags & ~(RA2A_AG_AGENT_SYNC | RA2A_AG_SKIP_RESET | RA2A_AG_B_TRANSPOSED))
        return fail(RA2A_EINVAL, "unknown flags");
    if (!a_shards || !gathered || !b || !c || !signals) return fail(RA2A_EINVAL, "NULL pointer");
    ra2a_heap* h = find_heap(a_shards);
    if (!h) return fail(RA2A_EINVAL, "a_shards is not inside a symmetric heap");
    if (h->world != W) return fail(RA2A_EINVAL, "W=%d but the heap has %d slices", W, h->world);
    if (!in_heap(h, gathered) || !in_heap(h, signals))
        return fail(RA2A_EINVAL, "gathered and signals must be inside the heap of a_shards");
    int nxcd = 1;
    int rc = RA2A_OK;
    bool agent = (flags & RA2A_AG_AGENT_SYNC) != 0;
    if (no_alloc) {
        if (!xcd_count_known(&nxcd)) agent = true;
    } else {
        rc = xcd_count(&nxcd);
        if (rc) return rc;
    }
    ra2a::AgGemmArgs a{};
    rc = plan_ag_gemm(W, rank, m_local, K, N, tile_rows, nxcd, agent, &a);
    if (rc) return rc;
    const size_t a_off = sym_offset(h, a_shards), g_off = sym_offset(h, gathered);
    const size_t s_off = sym_offset(h, signals);
    const size_t shard_bytes = (size_t)(m_local * K * 2), g_bytes = (size_t)W * shard_bytes;
    const int64_t nslots = ra2a::agg_queue_slot(a) + ra2a::kQueueSlots;
    const size_t s_bytes = (size_t)nslots * RA2A_SIG_STRIDE_BYTES;
    if (a_off % 16 || g_off % 16 || s_off % 8 || reinterpret_cast<uintptr_t>(b) % 16 ||
        reinterpret_cast<uintptr_t>(c) % 2)
        return fail(RA2A_EINVAL, "a_shards, gathered and b must be 16-byte aligned, signals 8, c 2");
    if (a_off + shard_bytes > h->stride || g_off + g_bytes > h->stride || s_off + s_bytes > h->stride)
        return fail(RA2A_EINVAL, "a shard, the gathered matrix or the signals cross the end of a slice");
    auto overlap = [](size_t o1, size_t n1, size_t o2, size_t n2) { return o1 < o2 + n2 && o2 < o1 + n1; };
    if (overlap(a_off, shard_bytes, g_off, g_bytes) || overlap(a_off, shard_bytes, s_off, s_bytes) ||
        overlap(g_off, g_bytes, s_off, s_bytes))
        return fail(RA2A_EINVAL, "a_shards, gathered and signals overlap");
    // XCD-local synchronisation reads G through the CU's L1, and a GEMM row block
    // waits only for the AllGather tiles of its own rows.  If a 128-byte line of G
    // held rows of two row blocks, a block could cache the line before the next
    // block's rows arrive and a later tile on the same CU read them stale.  Row
    // blocks start at g_off + (w*m_local + 256*mb)*K*2 bytes; unless every such
    // start is 128-byte aligned, synchronise device-wide (the acquire drops L1).
    if (a.sync == ra2a::kSyncXcd && (g_off % 128 != 0 || shard_bytes % 128 != 0))
        a.sync = ra2a::kSyncAgent;
    uint8_t* scr = nullptr;
    if (no_alloc) {
        rc = scratch_address(&scr);
        if (rc) return rc;
    } else {
        rc = ensure_err(h);
        if (rc) return rc;
    }
    a.base = h->base;
    a.stride = (int64_t)h->stride;
    a.a_off = (int64_t)a_off;
    a.g_off = (int64_t)g_off;
    a.sig_off = (int64_t)s_off;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (flags & RA2A_AG_B_TRANSPOSED) {
        a.bt = static_cast<const uint16_t*>(b);
    } else {
        // B^T into a workspace (the matrix cores take both operands k-contiguous)
        const size_t need = (size_t)(K * N * 2);
        uint16_t* bt = nullptr;
        if (no_alloc) {
            if (need > kScratchBtBytes)
                return fail(RA2A_EINVAL, "B^T of %zu bytes exceeds the %zu-byte scratch of the "
                                         "allocation-free entry point (pass B transposed)", need,
                            kScratchBtBytes);
            bt = reinterpret_cast<uint16_t*>(scr + kScratchErrBytes);
        } else {
            std::lock_guard<std::mutex> lk(h->mu);
            if (h->bt_bytes < need) {
                if (h->bt_ws) {
                    hipError_t e = hipDeviceSynchronize();  // earlier launches may still read it
                    if (e == hipSuccess) e = hipFree(h->bt_ws);
                    h->bt_ws = nullptr;
                    h->bt_bytes = 0;
                    if (e != hipSuccess) return hip_fail(e, "B^T workspace release");
                }
                void* p = nullptr;
                hipError_t e = hipMalloc(&p, need);
                if (e != hipSuccess) {
                    (void)hipGetLastError();
                    return fail(RA2A_ENOMEM, "B^T workspace of %zu bytes: %s", need, hipGetErrorString(e));
                }
                h->bt_ws = p;
                h->bt_bytes = need;
            }
            bt = static_cast<uint16_t*>(h->bt_ws);
        }
        hipError_t e = ra2a::launch_transpose_b(static_cast<const uint16_t*>(b), bt, K, N, st);
        if (e != hipSuccess) return hip_fail(e, "B transpose launch");
        a.bt = bt;
    }
    a.c = static_cast<uint16_t*>(c);
    a.err = no_alloc ? reinterpret_cast<uint32_t*>(scr) : h->err;
    a.timeout = timeout_ticks(h);
    int ncu = 0;
    rc = device_cus(&ncu);
    if (rc) return rc;
    int occ = 0;
    hipError_t he = ra2a::ag_gemm_blocks_per_cu(a.sync, &occ);
    if (he != hipSuccess) return hip_fail(he, "occupancy query");
    if (occ < 1) return fail(RA2A_EUNSUPPORTED, "the AllGather+GEMM kernel does not fit a compute unit");
    if (!(flags & RA2A_AG_SKIP_RESET)) {
        he = ra2a::launch_signal_reset(h->base, (int64_t)h->stride, W, (int64_t)s_off, nslots, st);
        if (he != hipSuccess) return hip_fail(he, "signal reset launch");
    }
    he = ra2a::launch_ag_gemm(a, occ * ncu, st);
    if (he != hipSuccess) return hip_fail(he, "AllGather+GEMM launch");
    return ok();
}

}  // namespace

RA2A_API int ra2a_ag_gemm(const void* a_shards, void* gathered, const void* b, void* c,
                          uint64_t* signals, int W, int rank, int64_t m_local, int64_t K, int64_t N,
                          int tile_rows, int flags, void* stream) {
    return ag_gemm_run(a_shards, gathered, b, c, signals, W, rank, m_local, K, N, tile_rows, flags,
                       stream, false);
}

RA2A_API int ra2a_ag_gemm_noalloc(const void* a_shards, void* gathered, const void* b, void* c,
                                  uint64_t* signals, int W, int rank, int64_t m_local, int64_t K,
                                  int64_t N, int tile_rows, int flags, void* stream) {
    NoAllocScope guard;
    return ag_gemm_run(a_shards, gathered, b, c, signals, W, rank, m_local, K, N, tile_rows, flags,
                       stream, true);
}

// ===========================================================================
// GEMM + ReduceScatter

namespace {

// bytes of the receive area: W slots of ntiles partial tiles (fp32 or bf16)
size_t gemm_rs_area(const ra2a::GemmRsArgs& a) { return (size_t)ra2a::grs_part_offset(a, a.W, 0); }

int plan_gemm_rs(int W, int64_t m, int64_t K, int64_t N, int nxcd, int flags,
                 ra2a::GemmRsArgs* a) {
    if (flags & ~(RA2A_RS_AGENT_SYNC | RA2A_RS_SKIP_RESET | RA2A_RS_BF16_PARTIALS))
        return fail(RA2A_EINVAL, "unknown flags");
    if (W < 1) return fail(RA2A_EINVAL, "W must be >= 1");
    if (m < 1 || K < 1 || N < 1) return fail(RA2A_EINVAL, "m, K and N must be >= 1");
    if (m % W) return fail(RA2A_EINVAL, "m=%lld must be divisible by W=%d (each rank receives m/W rows)",
                           (long long)m, W);
    if (K % 8) return fail(RA2A_EINVAL, "K must be a multiple of 8 (16-byte rows)");
    *a = ra2a::GemmRsArgs{};
    a->W = W;
    a->m = m;
    a->mj = m / W;
    a->K = K;
    a->N = N;
    a->ntm = (int)cdiv(a->mj, ra2a::kRsTileM);
    a->ntn = (int)cdiv(N, ra2a::kRsTileN);
    a->ntiles = a->ntm * a->ntn;
    a->nblocks = (int)cdiv(a->ntiles, ra2a::kRsBlock);
    a->NG = std::max(1, std::min(nxcd, ra2a::kNumXcd));
    a->dpg = (int)cdiv(W, a->NG);
    a->sync = ((flags & RA2A_RS_AGENT_SYNC) || nxcd > ra2a::kNumXcd) ? ra2a::kSyncAgent : ra2a::kSyncXcd;
    a->f32p = (flags & RA2A_RS_BF16_PARTIALS) ? 0 : 1;
    a->ntasks_dest = (int64_t)a->ntiles * W;
    if ((double)a->ntasks_dest * a->dpg >= 2147483647.0 - 65536.0)
        return fail(RA2A_EINVAL, "GEMM+ReduceScatter too large for 32-bit task indices");
    // a GEMM tile's operand rows and the receive area are addressed with 32-bit buffer offsets
    if ((double)ra2a::kRsTileN * K * 2 >= 4294967295.0 - 65536.0)
        return fail(RA2A_EINVAL, "K too large for 32-bit operand offsets");
    if ((double)W * a->ntiles * ra2a::kRsPartElems * (a->f32p ? 4 : 2) >= 4294967295.0 - 65536.0)
        return fail(RA2A_EINVAL, "receive area of 4 GiB or more per slice");
    return RA2A_OK;
}

}  // namespace

RA2A_API int ra2a_gemm_rs_sizes(int W, int64_t m, int64_t K, int64_t N, int flags,
                                int64_t* tile_slots, int64_t* queue_slots, size_t* partial_bytes) {
    ra2a::GemmRsArgs a{};
    int rc = plan_gemm_rs(W, m, K, N, ra2a::kNumXcd, flags, &a);
    if (rc) return rc;
    if (tile_slots) *tile_slots = (int64_t)a.ntiles * W;
    if (queue_slots) *queue_slots = ra2a::kQueueSlots;
    if (partial_bytes) *partial_bytes = gemm_rs_area(a);
    return ok();
}

RA2A_API int ra2a_gemm_rs(const void* x1, const void* x2t, void* partial, void* out,
                          uint64_t* signals, int W, int64_t m, int64_t K, int64_t N, int flags,
                          void* stream) {
    if (flags & ~(RA2A_RS_AGENT_SYNC | RA2A_RS_SKIP_RESET | RA2A_RS_BF16_PARTIALS))
        return fail(RA2A_EINVAL, "unknown flags");
    if (!x1 || !x2t || !partial || !out || !signals) return fail(RA2A_EINVAL, "NULL pointer");
    ra2a_heap* h = find_heap(x1);
    if (!h) return fail(RA2A_EINVAL, "x1 is not inside a symmetric heap");
    if (h->world != W) return fail(RA2A_EINVAL, "W=%d but the heap has %d slices", W, h->world);
    if (!in_heap(h, x2t) || !in_heap(h, partial) || !in_heap(h, out) || !in_heap(h, signals))
        return fail(RA2A_EINVAL, "x2t, partial, out and signals must be inside the heap of x1");
    // every argument check before the first device query
    ra2a::GemmRsArgs a{};
    int rc = plan_gemm_rs(W, m, K, N, ra2a::kNumXcd, flags, &a);
    if (rc) return rc;
    const size_t o_a = sym_offset(h, x1), o_b = sym_offset(h, x2t), o_p = sym_offset(h, partial);
    const size_t o_o = sym_offset(h, out), o_s = sym_offset(h, signals);
    const size_t n_a = (size_t)(m * K * 2), n_b = (size_t)(N * K * 2);
    const size_t n_p = gemm_rs_area(a), n_o = (size_t)(a.mj * N * 2);
    const int64_t nslots = ra2a::grs_queue_slot(a) + ra2a::kQueueSlots;
    const size_t n_s = (size_t)nslots * RA2A_SIG_STRIDE_BYTES;
    if (o_a % 16 || o_b % 16 || o_p % 16 || o_o % 8 || o_s % 8)
        return fail(RA2A_EINVAL, "x1, x2t and partial must be 16-byte aligned, out and signals 8");
    const size_t offs[5] = {o_a, o_b, o_p, o_o, o_s}, lens[5] = {n_a, n_b, n_p, n_o, n_s};
    for (int i = 0; i < 5; ++i) {
        if (offs[i] + lens[i] > h->stride)
            return fail(RA2A_EINVAL, "an operand, the receive area, out or the signals cross the "
                                     "end of a slice");
        for (int k2 = 0; k2 < i; ++k2)
            if (offs[i] < offs[k2] + lens[k2] && offs[k2] < offs[i] + lens[i])
                return fail(RA2A_EINVAL, "x1, x2t, partial, out and signals must not overlap");
    }
    int nxcd = 1;
    rc = xcd_count(&nxcd);
    if (rc) return rc;
    rc = plan_gemm_rs(W, m, K, N, nxcd, flags, &a);  // the queues of this device's XCDs
    if (rc) return rc;
    rc = ensure_err(h);
    if (rc) return rc;
    a.base = h->base;
    a.stride = (int64_t)h->stride;
    a.a_off = (int64_t)o_a;
    a.bt_off = (int64_t)o_b;
    a.p_off = (int64_t)o_p;
    a.out_off = (int64_t)o_o;
    a.sig_off = (int64_t)o_s;
    a.err = h->err;
    a.timeout = timeout_ticks(h);
    int ncu = 0;
    rc = device_cus(&ncu);
    if (rc) return rc;
    int occ = 0;
    hipError_t he = ra2a::gemm_rs_blocks_per_cu(a.sync, a.f32p != 0, &occ);
    if (he != hipSuccess) return hip_fail(he, "occupancy query");
    if (occ < 1) return fail(RA2A_EUNSUPPORTED, "the GEMM+ReduceScatter kernel does not fit a compute unit");
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (!(flags & RA2A_RS_SKIP_RESET)) {
        he = ra2a::launch_signal_reset(h->base, (int64_t)h->stride, W, (int64_t)o_s, nslots, st);
        if (he != hipSuccess) return hip_fail(he, "signal reset launch");
    }
    he = ra2a::launch_gemm_rs(a, occ * ncu, st);
    if (he != hipSuccess) return hip_fail(he, "GEMM+ReduceScatter launch");
    return ok();
}

RA2A_API int ra2a_debug_gemm_rs_plan(int W, int64_t m, int64_t K, int64_t N, int num_xcd,
                                     int64_t* tasks_per_group) {
    ra2a::GemmRsArgs a{};
    int rc = plan_gemm_rs(W, m, K, N, std::max(1, num_xcd), 0, &a);
    if (rc) return rc;
    // every destination's queue: each (source, tile) task exactly once, and the
    // receiver's task of a tile (r == j, which waits) after the W - 1 it waits for
    for (int g = 0; g < a.NG; ++g) {
        const int64_t total = a.ntasks_dest * a.dpg;
        std::vector<int> done((size_t)W * a.ntiles * W, 0);
        for (int64_t pos = 0; pos < total; ++pos) {
            const ra2a::RsTask t = ra2a::grs_group_task(a, g, pos);
            if (t.j < 0 || t.tile < 0 || t.tile >= a.ntiles || t.r < 0 || t.r >= W ||
                t.j % a.NG != g)
                return fail(RA2A_EINVAL, "group %d position %lld: task out of range", g, (long long)pos);
            if (t.j >= W) continue;  // padding of the last group
            if (t.r == t.j)
                for (int r = 0; r < W; ++r)
                    if (r != t.j && !done[((size_t)t.j * a.ntiles + t.tile) * W + r])
                        return fail(RA2A_EINVAL, "group %d position %lld: the receiver's task of tile %d "
                                    "waits for a task queued after it", g, (long long)pos, t.tile);
            int& d = done[((size_t)t.j * a.ntiles + t.tile) * W + t.r];
            if (d++) return fail(RA2A_EINVAL, "task (j=%d, tile=%d, r=%d) twice", t.j, t.tile, t.r);
        }
        for (int j = g; j < W; j += a.NG)
            for (int t = 0; t < a.ntiles; ++t)
                for (int r = 0; r < W; ++r)
                    if (!done[((size_t)j * a.ntiles + t) * W + r])
                        return fail(RA2A_EINVAL, "a task is missing");
    }
    if (tasks_per_group) *tasks_per_group = a.ntasks_dest * a.dpg;
    return ok();
}

// ===========================================================================
// Variable-size AllToAll

namespace {

// Default bytes per data chunk.  Measured on 7.5 GB AllToAlls (W = 8, rows of 4096,
// 7168 and 14336 bytes): chunks of 40 / 44 / 48 / 64 / 256 KiB run at 72 / 75 / 74
// / 68 / 64 % of 8 TB/s, and below 40 KiB the per-chunk claim, wait and signal
// take over.
constexpr int64_t kA2vDefaultChunk = 44 << 10;

int check_a2v_shape(int W, int64_t row_bytes, int64_t in_rows, int64_t out_rows, int64_t* chunk) {
    if (W < 1 || W > ra2a::kA2vMaxW) return fail(RA2A_EINVAL, "W must be in 1..%d", ra2a::kA2vMaxW);
    if (row_bytes < 1) return fail(RA2A_EINVAL, "row_bytes must be >= 1");
    if (in_rows < 0 || out_rows < 0) return fail(RA2A_EINVAL, "row capacities must be >= 0");
    if ((double)in_rows * row_bytes >= 4.6e18 || (double)out_rows * row_bytes >= 4.6e18)
        return fail(RA2A_EINVAL, "buffers too large");
    if (*chunk == 0) *chunk = kA2vDefaultChunk;
    if (*chunk < 16 || *chunk % 16) return fail(RA2A_EINVAL, "chunk_bytes must be a positive multiple of 16");
    // the queue positions of one launch: 3W + the chunks of every segment (each at most in_rows rows)
    const double chunks = (double)W * W * ((double)in_rows * row_bytes / (double)*chunk + 1.0);
    if (3.0 * W + chunks >= 9.0e18) return fail(RA2A_EINVAL, "too many chunks");
    return RA2A_OK;
}

int a2v_vector(int64_t row_bytes) { return row_bytes % 16 == 0 ? 16 : row_bytes % 4 == 0 ? 4 : 1; }

}  // namespace

RA2A_API int ra2a_alltoallv_signal_slots(int W, int64_t* slots) {
    if (W < 1 || W > ra2a::kA2vMaxW) return fail(RA2A_EINVAL, "W must be in 1..%d", ra2a::kA2vMaxW);
    if (slots) *slots = ra2a::a2v_slots(W);
    return ok();
}

RA2A_API int ra2a_alltoallv(const void* in, const int64_t* send_counts, void* out, int64_t* recv_counts,
                            uint64_t* signals, int W, int64_t row_bytes, int64_t in_rows,
                            int64_t out_rows, int64_t chunk_bytes, int flags, void* stream) {
    if (flags & ~RA2A_A2V_SKIP_RESET) return fail(RA2A_EINVAL, "unknown flags");
    if (!in || !send_counts || !out || !recv_counts || !signals) return fail(RA2A_EINVAL, "NULL pointer");
    int64_t chunk = chunk_bytes;
    int rc = check_a2v_shape(W, row_bytes, in_rows, out_rows, &chunk);
    if (rc) return rc;
    ra2a_heap* h = find_heap(in);
    if (!h) return fail(RA2A_EINVAL, "in is not inside a symmetric heap");
    if (h->world != W) return fail(RA2A_EINVAL, "W=%d but the heap has %d slices", W, h->world);
    if (!in_heap(h, send_counts) || !in_heap(h, out) || !in_heap(h, recv_counts) || !in_heap(h, signals))
        return fail(RA2A_EINVAL, "send_counts, out, recv_counts and signals must be inside the heap of in");
    const size_t offs[5] = {sym_offset(h, in), sym_offset(h, send_counts), sym_offset(h, out),
                            sym_offset(h, recv_counts), sym_offset(h, signals)};
    const size_t lens[5] = {(size_t)(in_rows * row_bytes), (size_t)W * 8u, (size_t)(out_rows * row_bytes),
                            (size_t)(W + 1) * 8u, (size_t)ra2a::a2v_slots(W) * RA2A_SIG_STRIDE_BYTES};
    if (offs[0] % 16 || offs[2] % 16) return fail(RA2A_EINVAL, "in and out must be 16-byte aligned");
    if (offs[1] % 8 || offs[3] % 8 || offs[4] % 8)
        return fail(RA2A_EINVAL, "send_counts, recv_counts and signals must be 8-byte aligned");
    for (int i = 0; i < 5; ++i) {
        if (offs[i] + lens[i] > h->stride)
            return fail(RA2A_EINVAL, "a buffer crosses the end of a slice");
        for (int k = 0; k < i; ++k)
            if (lens[i] && lens[k] && offs[i] < offs[k] + lens[k] && offs[k] < offs[i] + lens[i])
                return fail(RA2A_EINVAL, "in, send_counts, out, recv_counts and signals must not overlap");
    }
    rc = ensure_err(h);
    if (rc) return rc;
    ra2a::A2vArgs a{};
    a.base = h->base;
    a.stride = (int64_t)h->stride;
    a.in_off = (int64_t)offs[0];
    a.cnt_off = (int64_t)offs[1];
    a.out_off = (int64_t)offs[2];
    a.rc_off = (int64_t)offs[3];
    a.sig_off = (int64_t)offs[4];
    a.err = h->err;
    a.timeout = timeout_ticks(h);
    a.W = W;
    a.row_bytes = row_bytes;
    a.in_rows = in_rows;
    a.out_rows = out_rows;
    a.chunk = chunk;
    const int V = a2v_vector(row_bytes);
    int ncu = 0;
    rc = device_cus(&ncu);
    if (rc) return rc;
    int occ = 0;
    hipError_t he = ra2a::alltoallv_blocks_per_cu(V, &occ);
    if (he != hipSuccess) return hip_fail(he, "occupancy query");
    if (occ < 1) return fail(RA2A_EUNSUPPORTED, "the AllToAll kernel does not fit a compute unit");
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (!(flags & RA2A_A2V_SKIP_RESET)) {
        he = ra2a::launch_signal_reset(h->base, (int64_t)h->stride, W, (int64_t)offs[4],
                                       ra2a::a2v_slots(W), st);
        if (he != hipSuccess) return hip_fail(he, "signal reset launch");
    }
    he = ra2a::launch_alltoallv(a, V, std::min(occ, 4) * ncu, st);
    if (he != hipSuccess) return hip_fail(he, "AllToAll launch");
    return ok();
}

RA2A_API int ra2a_debug_alltoallv_emulate(int W, int64_t row_bytes, int64_t in_rows, int64_t out_rows,
                                          int64_t chunk_bytes, const void* const* in,
                                          const int64_t* send_counts, void* const* out,
                                          int64_t* recv_counts, uint64_t* signals, uint32_t* err_word,
                                          int64_t* tasks) {
    int64_t chunk = chunk_bytes;
    int rc = check_a2v_shape(W, row_bytes, in_rows, out_rows, &chunk);
    if (rc) return rc;
    if (!in || !send_counts || !out || !recv_counts || !signals || !err_word)
        return fail(RA2A_EINVAL, "NULL pointer");
    const int n = W * W;
    const int64_t S = ra2a::a2v_slots(W);
    // the kernel's own decode: usable counts, chunk table, queue positions
    std::vector<int64_t> cnt(send_counts, send_counts + n);
    std::vector<int> rank_ok((size_t)W);
    for (int r = 0; r < W; ++r) rank_ok[(size_t)r] = ra2a::a2v_rank_ok(W, in_rows, cnt.data() + r * W) ? 1 : 0;
    for (int i = 0; i < n; ++i)
        if (!rank_ok[(size_t)(i / W)]) cnt[(size_t)i] = 0;
    std::vector<int64_t> first((size_t)n + 1, 0);
    for (int p = 0; p < n; ++p) {
        const int r = p / W;
        first[(size_t)p + 1] = first[(size_t)p] +
                               ra2a::a2v_chunks(cnt[(size_t)(r * W + ra2a::a2v_dest(W, r, p - r * W))], row_bytes, chunk);
    }
    std::memset(signals, 0, sizeof(uint64_t) * (size_t)(W * S));
    auto sig = [&](int slice, int64_t slot) -> uint64_t& { return signals[(size_t)(slice * S + slot)]; };
    const int64_t total = ra2a::a2v_total(W, first.data());
    std::vector<int64_t> seen_chunks((size_t)n, 0);
    for (int64_t pos = 0; pos < total; ++pos) {
        const ra2a::A2vTask t = ra2a::a2v_task(W, first.data(), pos);
        if (t.kind == 0) {
            for (int j = 0; j < W; ++j) recv_counts[(size_t)(j * (W + 1) + t.r)] = cnt[(size_t)(t.r * W + j)];
            if (!rank_ok[(size_t)t.r]) *err_word |= ra2a::kErrCounts;
            for (int j = 0; j < W; ++j) sig(j, ra2a::a2v_count_slot()) += 1;
        } else if (t.kind == 1) {
            if (sig(t.j, ra2a::a2v_count_slot()) != (uint64_t)W)
                return fail(RA2A_EINVAL, "position %lld: offset task of %d waits for counts queued after it",
                            (long long)pos, t.j);
            int64_t run = 0;
            for (int r = 0; r < W; ++r) {
                sig(r, ra2a::a2v_offset_slot(t.j)) = (uint64_t)run + 1u;
                run += recv_counts[(size_t)(t.j * (W + 1) + r)];
            }
        } else if (t.kind == 2) {
            if (t.r < 0 || t.r >= W || t.j < 0 || t.j >= W) return fail(RA2A_EINVAL, "chunk task out of range");
            const uint64_t o = sig(t.r, ra2a::a2v_offset_slot(t.j));
            if (o == 0)
                return fail(RA2A_EINVAL, "position %lld: chunk waits for an offset queued after it", (long long)pos);
            const int64_t rows = cnt[(size_t)(t.r * W + t.j)];
            const int64_t nch = ra2a::a2v_chunks(rows, row_bytes, chunk);
            if (t.c < 0 || t.c >= nch || t.c != seen_chunks[(size_t)(t.r * W + t.j)]++)
                return fail(RA2A_EINVAL, "chunk %lld of (%d, %d) out of order", (long long)t.c, t.r, t.j);
            const int64_t dst_row = (int64_t)o - 1;
            if (dst_row >= 0 && rows <= out_rows && dst_row <= out_rows - rows) {
                int64_t lo, hi;
                ra2a::a2v_chunk_range(rows, row_bytes, chunk, t.c, &lo, &hi);
                const int64_t src_row = ra2a::a2v_send_offset(W, cnt.data(), t.r, t.j);
                std::memcpy(static_cast<uint8_t*>(out[t.j]) + dst_row * row_bytes + lo,
                            static_cast<const uint8_t*>(in[t.r]) + src_row * row_bytes + lo, (size_t)(hi - lo));
            } else {
                *err_word |= ra2a::kErrOverflow;
            }
            if (++sig(t.j, ra2a::a2v_chunk_slot(W, t.r)) == (uint64_t)nch) sig(t.j, ra2a::a2v_arrival_slot(W)) += 1;
        } else if (t.kind == 3) {
            if (sig(t.j, ra2a::a2v_arrival_slot(W)) != (uint64_t)W)
                return fail(RA2A_EINVAL, "position %lld: receive task of %d waits for data queued after it",
                            (long long)pos, t.j);
            int64_t sum = 0;
            for (int r = 0; r < W; ++r) sum += recv_counts[(size_t)(t.j * (W + 1) + r)];
            recv_counts[(size_t)(t.j * (W + 1) + W)] = sum;
        } else {
            return fail(RA2A_EINVAL, "position %lld decodes to no task", (long long)pos);
        }
    }
    for (int p = 0; p < n; ++p) {
        const int r = p / W, j = p % W;
        if (seen_chunks[(size_t)p] != ra2a::a2v_chunks(cnt[(size_t)p], row_bytes, chunk))
            return fail(RA2A_EINVAL, "segment (%d, %d): not every chunk queued", r, j);
    }
    sig(0, ra2a::a2v_queue_slot(W)) = (uint64_t)total;
    if (tasks) *tasks = total;
    return ok();
}

RA2A_API int ra2a_debug_ag_gemm_plan(int W, int rank, int64_t m_local, int64_t K, int64_t N,
                                     int tile_rows, int num_xcd, int64_t* tasks_per_group) {
    ra2a::AgGemmArgs a{};
    int rc = plan_ag_gemm(W, rank, m_local, K, N, tile_rows, num_xcd, false, &a);
    if (rc) return rc;
    if (tasks_per_group) *tasks_per_group = a.ntasks_shard * a.spg;
    // every part of every shard exactly once, rows covering the shard; every GEMM
    // tile exactly once and after every part of the tiles it waits for
    for (int g = 0; g < a.NG; ++g) {
        const int64_t total = a.ntasks_shard * a.spg;
        for (int si = 0; si < a.spg; ++si) {
            const int w = g + si * a.NG;
            std::vector<int> row_hits((size_t)m_local, 0);
            std::vector<int> parts_seen((size_t)a.ntiles, 0);
            std::vector<int> gemm_seen((size_t)a.nmb * a.ncol, 0);
            for (int64_t pos = (int64_t)si * a.ntasks_shard; pos < (int64_t)(si + 1) * a.ntasks_shard; ++pos) {
                const ra2a::AgTask t = ra2a::agg_task_of(a, g, pos);
                if (t.w != w) return fail(RA2A_EINVAL, "group %d position %lld: shard %d, expected %d", g, (long long)pos, t.w, w);
                if (!t.gemm) {
                    if (t.tile < 0 || t.tile >= a.ntiles || t.part < 0 || t.part >= ra2a::agg_parts_of_tile(a, t.tile) || t.rows < 1)
                        return fail(RA2A_EINVAL, "bad AllGather part (tile %d part %d rows %lld)", t.tile, t.part, (long long)t.rows);
                    if (t.row0 < (int64_t)t.tile * a.tile_rows || t.row0 + t.rows > std::min<int64_t>((int64_t)(t.tile + 1) * a.tile_rows, m_local))
                        return fail(RA2A_EINVAL, "AllGather part straddles its tile");
                    for (int64_t r = t.row0; r < t.row0 + t.rows; ++r) row_hits[(size_t)r]++;
                    parts_seen[(size_t)t.tile]++;
                } else {
                    if (t.mb < 0 || t.mb >= a.nmb || t.nb < 0 || t.nb >= a.ncol)
                        return fail(RA2A_EINVAL, "bad GEMM tile (%d, %d)", t.mb, t.nb);
                    gemm_seen[(size_t)t.mb * a.ncol + t.nb]++;
                    int first, last;
                    ra2a::agg_block_tiles(a, t.mb, &first, &last);
                    if (first < 0 || last > a.ntiles || first >= last)
                        return fail(RA2A_EINVAL, "GEMM row block %d waits for tiles [%d, %d)", t.mb, first, last);
                    for (int x = first; x < last; ++x)
                        if (parts_seen[(size_t)x] != ra2a::agg_parts_of_tile(a, x))
                            return fail(RA2A_EINVAL, "group %d position %lld: GEMM tile (%d, %d) waits for tile %d "
                                        "whose parts are queued after it", g, (long long)pos, t.mb, t.nb, x);
                    // its rows must lie inside the tiles it waits for
                    const int64_t r0 = (int64_t)t.mb * ra2a::kGemmBM;
                    const int64_t r1 = std::min<int64_t>(r0 + ra2a::kGemmBM, m_local);
                    if (r0 < (int64_t)first * a.tile_rows || r1 > std::min<int64_t>((int64_t)last * a.tile_rows, m_local))
                        return fail(RA2A_EINVAL, "GEMM row block %d is not covered by tiles [%d, %d)", t.mb, first, last);
                }
            }
            for (int x : row_hits)
                if (x != 1) return fail(RA2A_EINVAL, "shard %d: AllGather parts do not cover its rows once", w);
            for (int x : gemm_seen)
                if (x != 1) return fail(RA2A_EINVAL, "shard %d: GEMM tiles are not each queued once", w);
        }
        (void)total;
    }
    return ok();
}

// ===========================================================================
// diagnostics

RA2A_API int ra2a_check(const ra2a_heap_t* h) {
    if (!h) return fail(RA2A_EINVAL, "heap must be non-NULL");
    hipError_t e = hipDeviceSynchronize();
    if (e != hipSuccess) return hip_fail(e, "hipDeviceSynchronize");
    // the heap's error word, and the current device's scratch error word (used by
    // the allocation-free entry points), if either exists; both read and cleared
    uint32_t w = 0;
    uint32_t* words[2] = {h->err, nullptr};
    {
        int dev = 0;
        if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < kMaxDevices) {
            std::lock_guard<std::mutex> g(g_scratch_mu);
            words[1] = reinterpret_cast<uint32_t*>(g_scratch[dev]);
        }
    }
    for (uint32_t* word : words) {
        if (!word) continue;
        uint32_t x = 0;
        e = hipMemcpy(&x, word, sizeof x, hipMemcpyDeviceToHost);
        if (e != hipSuccess) return hip_fail(e, "reading an error word");
        if (x) {
            e = hipMemset(word, 0, sizeof x);
            if (e != hipSuccess) return hip_fail(e, "clearing an error word");
        }
        w |= x;
    }
    if (w) {
        if (w & (ra2a::kErrCounts | ra2a::kErrOverflow))
            return fail(RA2A_EDATA, "device-side data check failed (error word 0x%x:%s%s%s)", w,
                        (w & ra2a::kErrCounts) ? " a sender's counts were unusable" : "",
                        (w & ra2a::kErrOverflow) ? " a destination received more rows than it holds" : "",
                        (w & ra2a::kErrTimeout) ? " a bounded wait timed out" : "");
        return fail(RA2A_ETIMEOUT, "a bounded device-side wait timed out (error word 0x%x)", w);
    }
    return ok();
}

RA2A_API const char* ra2a_last_error(void) { return g_err.c_str(); }

RA2A_API int ra2a_version(void) { return 200; }

// ===========================================================================
// host emulation of the pipelined combine's address arithmetic

namespace {

// The offsets of vectors [lo, hi) of a row plan as the kernels' threads walk
// them (thread t: lo + t, lo + t + 256, ... with a cursor), each checked against
// the direct decomposition of its index.
int walk_plan(const ra2a::RowPlan& p, int V, int lo, int hi,
              std::vector<std::pair<int64_t, int64_t>>* out) {
    out->clear();
    if (hi <= lo) return RA2A_OK;
    const int vpr = p.run / V;
    if (vpr < 1 || p.run % V) return fail(RA2A_EINVAL, "row of %d bytes is not a multiple of %d", p.run, V);
    for (int t = 0; t < ra2a::kThreads && lo + t < hi; ++t) {
        ra2a::PlanCursor c = ra2a::cursor_start(p, V, vpr, (uint32_t)(lo + t), ra2a::kThreads);
        for (int idx = lo + t; idx < hi; idx += ra2a::kThreads) {
            int64_t so, dofs;
            ra2a::plan_offsets(p, V, vpr, (uint32_t)idx, &so, &dofs);
            if (so != c.so || dofs != c.dofs)
                return fail(RA2A_EINVAL, "cursor at vector %d: (%lld, %lld), direct (%lld, %lld)", idx,
                            (long long)c.so, (long long)c.dofs, (long long)so, (long long)dofs);
            out->push_back({so, dofs});
            ra2a::cursor_advance(c, p, vpr);
        }
    }
    return RA2A_OK;
}

}  // namespace

RA2A_API int ra2a_debug_emulate_pipelined(const void* const* in, void* const* out,
                                          uint64_t* const* signals, int W, int64_t S, int64_t H,
                                          int64_t D, int dtype, const ra2a_opts_t* opts,
                                          int num_cus, int blocks_per_cu) {
    const int e0 = elem_bytes(dtype);
    if (!e0) return fail(RA2A_EINVAL, "unknown dtype %d", dtype);
    if (W < 1 || S < 1 || H < 1 || D < 1 || !in || !out || num_cus < 1 || blocks_per_cu < 1)
        return fail(RA2A_EINVAL, "bad arguments");
    Plan pl{};
    int rc = make_plan(W, S, H, D, e0, opts, &pl);
    if (rc) return rc;
    auto al = [](int64_t x) { return (x + 255) / 256 * 256; };
    const int64_t nb = S * (int64_t)W * H * D * e0;
    const int64_t in_off = 0, out_off = al(nb), stg_off = al(out_off + nb);
    const int64_t sig_off = al(stg_off + pl.ring_bytes);
    const int64_t nsig = pl.regionA + pl.regionB + ra2a::kQueueSlots + ra2a::kResetFlags;
    const int64_t stride = al(sig_off + nsig * RA2A_SIG_STRIDE_BYTES);
    if ((double)stride * W > 16.0e9) return fail(RA2A_EINVAL, "too large to emulate");
    ra2a::PipeArgs a{};
    int V = 16, grid = 0;
    rc = prepare_pipelined(W, S, H, D, e0, pl, opts, stride, (size_t)in_off, (size_t)out_off,
                           (size_t)stg_off, (size_t)sig_off, num_cus, blocks_per_cu,
                           ra2a::kNumXcd, &a, &V, &grid);
    if (rc) return rc;
    std::vector<uint8_t> heap((size_t)(stride * W), 0xCD);
    for (int r = 0; r < W; ++r) {
        std::memcpy(&heap[(size_t)(r * stride + in_off)], in[r], (size_t)nb);
        std::memset(&heap[(size_t)(r * stride + sig_off)], 0, (size_t)(nsig * RA2A_SIG_STRIDE_BYTES));
    }
    auto u64 = [&](int64_t off) { return reinterpret_cast<uint64_t*>(&heap[(size_t)off]); };
    auto inside = [&](int64_t off, int64_t len, int slice, int64_t region, int64_t rlen) {
        const int64_t lo = (int64_t)slice * stride + region;
        return off >= lo && off + len <= lo + rlen;
    };

    {
        // every stream belongs to exactly one group
        std::vector<int> own((size_t)a.nstreams, 0);
        for (int g = 0; g < a.NG; ++g) {
            const ra2a::GroupStreams gs = ra2a::group_streams(a, g);
            for (int k = 0; k < gs.ns; ++k) own[(size_t)(gs.start + k)]++;
        }
        for (int x : own)
            if (x != 1) return fail(RA2A_EINVAL, "stream groups do not partition the streams");
    }

    const bool add = a.protocol == ra2a::kSigAdd;
    const int64_t sigA_len = pl.regionA * RA2A_SIG_STRIDE_BYTES;
    if (pl.rows) {
        // Row units as the kernel runs them: every unit once in its global order;
        // each fills whole output rows, adds 1 to its block's arrival counter, and
        // the unit that completes the block marks its signal tiles.  Every output
        // row must be written by exactly one unit.
        const int64_t total = ra2a::total_row_units(a);
        if (total != a.nunits) return fail(RA2A_EINVAL, "row unit count mismatch");
        std::vector<uint8_t> rowhit((size_t)(W * S), 0);
        const int64_t sigB_len = pl.regionB * RA2A_SIG_STRIDE_BYTES;
        for (int64_t u = 0; u < total; ++u) {
            const ra2a::RowUnit q = ra2a::row_unit(a, u);
            if (q.j < 0 || q.j >= W || q.b < 0 || q.b >= a.nbs || q.rows < 1 || q.k < 0 ||
                q.k >= q.nub)
                return fail(RA2A_EINVAL, "row unit %lld out of range", (long long)u);
            const int64_t s0 = (int64_t)q.b * a.BS + (int64_t)q.k * a.KU;
            for (int64_t t = s0; t < s0 + q.rows; ++t) {
                if (t >= S || t >= (int64_t)(q.b + 1) * a.BS)
                    return fail(RA2A_EINVAL, "row unit %lld leaves its S-block", (long long)u);
                rowhit[(size_t)(q.j * S + t)]++;
            }
            std::vector<std::pair<int64_t, int64_t>> offs;
            rc = walk_plan(q.pl, V, 0, ra2a::plan_vectors(q.pl, V), &offs);
            if (rc) return rc;
            // the dispatch stores to every destination r through r's own descriptor,
            // which covers the unit's rows of out_r (rows * run bytes)
            const int64_t run_b = (int64_t)q.pl.run;
            for (const auto& o : offs) {
                const int64_t so = q.src + o.first;
                const int r = (int)(so / stride);
                if (r < 0 || r >= W || !inside(so, V, r, in_off, nb))
                    return fail(RA2A_EINVAL, "row unit reads outside every input");
                const int64_t dabs = q.dst + o.second;
                const int rd = (int)(dabs / stride);
                if (pl.inverse) {
                    const int64_t rel = dabs - (int64_t)rd * stride - q.dst;
                    if (rd < 0 || rd >= W || rel < 0 || rel + V > (int64_t)q.rows * run_b)
                        return fail(RA2A_EINVAL, "row unit store outside its descriptor's range");
                } else if (o.second < 0 || o.second + V > (int64_t)ra2a::plan_span(q.pl)) {
                    return fail(RA2A_EINVAL, "row unit store outside its descriptor's range");
                }
                if (!inside(dabs, V, pl.inverse ? rd : q.j, out_off, nb))
                    return fail(RA2A_EINVAL, "row unit writes outside out of rank %d", rd);
                std::memcpy(&heap[(size_t)dabs], &heap[(size_t)so], (size_t)V);
            }
            if (!inside(q.cnt, 8, q.j, sig_off + sigA_len, sigB_len))
                return fail(RA2A_EINVAL, "row unit counter outside region B");
            *u64(q.cnt) += 1;
            if (*u64(q.cnt) > (uint64_t)q.nub)
                return fail(RA2A_EINVAL, "block counter beyond its unit count");
            if (*u64(q.cnt) == (uint64_t)q.nub)  // the unit that completes the block
                for (int d = 0; d < q.nd; ++d)
                    for (int k = 0; k < q.nsig; ++k) {
                        const int64_t sg = q.sig + (int64_t)d * stride + (int64_t)k * q.sig_step;
                        const int rs = q.nd == 1 ? q.j : d;
                        if (!inside(sg, 8, rs, sig_off, sigA_len))
                            return fail(RA2A_EINVAL, "row unit signal outside region A");
                        *u64(sg) = add ? *u64(sg) + (uint64_t)W : 1;
                    }
        }
        for (uint8_t x : rowhit)
            if (x != 1) return fail(RA2A_EINVAL, "row units do not write every output row once");
    } else if (pl.direct) {
        // Direct mode as the kernel runs it: every piece once in its global order,
        // no waits, no hand-back counters.
        const int64_t total = ra2a::total_pieces(a);
        std::vector<int64_t> seen((size_t)a.nstreams * a.nbs * W, 0);  // rows per (stream, S-block, source)
        for (int64_t gp = 0; gp < total; ++gp) {
            const ra2a::Piece p = ra2a::direct_piece(a, gp);
            if (p.sid < 0 || p.sid >= a.nstreams || p.b < 0 || p.b >= a.nbs || p.r < 0 || p.r >= W ||
                p.sub < 0 || p.sub >= p.nsub || p.nsub > a.nsub || p.pl.A < 1)
                return fail(RA2A_EINVAL, "direct piece %lld out of range", (long long)gp);
            seen[(size_t)(((int64_t)p.sid * a.nbs + p.b) * W + p.r)] += p.pl.A;
            std::vector<std::pair<int64_t, int64_t>> offs;
            rc = walk_plan(p.pl, V, 0, ra2a::plan_vectors(p.pl, V), &offs);
            if (rc) return rc;
            for (const auto& o : offs) {
                if (o.second < 0 || o.second + V > (int64_t)ra2a::plan_span(p.pl))
                    return fail(RA2A_EINVAL, "piece store outside its descriptor's range");
                if (!inside(p.src + o.first, V, p.r, in_off, nb))
                    return fail(RA2A_EINVAL, "piece reads outside in of rank %d", p.r);
                if (!inside(p.dst + o.second, V, p.j, out_off, nb))
                    return fail(RA2A_EINVAL, "piece writes outside out of rank %d", p.j);
                std::memcpy(&heap[(size_t)(p.dst + o.second)], &heap[(size_t)(p.src + o.first)], (size_t)V);
            }
            bool last = true;  // one piece per tile and source: it signals itself
            uint64_t val = 1;
            if (a.nsub > 1) {  // count the arrival; the last one signals for all
                if (!inside(p.cnt, 8, p.j, sig_off + sigA_len, pl.regionB * RA2A_SIG_STRIDE_BYTES))
                    return fail(RA2A_EINVAL, "piece counter outside region B");
                *u64(p.cnt) += 1;
                if (*u64(p.cnt) > p.cnt_need) return fail(RA2A_EINVAL, "tile counter beyond its need");
                last = *u64(p.cnt) == p.cnt_need;
                val = add ? (uint64_t)W : 1;
            }
            for (int k = 0; k < p.nsig && last; ++k) {
                const int64_t sg = p.sig + k * p.sig_step;
                if (!inside(sg, 8, p.j, sig_off, sigA_len))
                    return fail(RA2A_EINVAL, "piece signal outside region A");
                *u64(sg) = add ? *u64(sg) + val : 1;
            }
        }
        // every (stream, S-block, source) moved each of its rows exactly once
        for (int sid = 0; sid < a.nstreams; ++sid)
            for (int b = 0; b < a.nbs; ++b)
                for (int r = 0; r < W; ++r)
                    if (seen[(size_t)(((int64_t)sid * a.nbs + b) * W + r)] !=
                        std::min<int64_t>(a.BS, S - (int64_t)b * a.BS))
                        return fail(RA2A_EINVAL, "direct schedule does not move every row once");
    }
    // Staged mode: each group's queue run strictly in queue order, one task at a
    // time: every wait must already hold when its task comes up (the kernel's
    // deadlock-freedom argument), and the queue must hold every piece and item once.
    for (int g = 0; g < a.NG && !pl.direct; ++g) {
        const ra2a::GroupQueue Q = ra2a::group_queue(a, g);
        const int64_t npieces = ra2a::group_pieces(a, g);
        const int64_t nitems = ra2a::group_items(a, g);
        if (Q.total != npieces + nitems || Q.L < 0 || Q.L > Q.ntiles)
            return fail(RA2A_EINVAL, "group %d: queue of %lld tasks for %lld pieces and %lld items",
                        g, (long long)Q.total, (long long)npieces, (long long)nitems);
        std::vector<uint8_t> cov_p((size_t)npieces, 0), cov_i((size_t)nitems, 0);
        for (int64_t pos = 0; pos < Q.total; ++pos) {
            int64_t idx = -1;
            if (ra2a::task_of(Q, pos, &idx)) {
                if (idx < 0 || idx >= npieces) return fail(RA2A_EINVAL, "queue piece out of range");
                cov_p[(size_t)idx]++;
                const ra2a::Piece p = ra2a::piece_of(a, g, idx);
                if (p.b < 0 || p.b >= a.nbs) return fail(RA2A_EINVAL, "piece S-block out of range");
                if (p.b >= a.R) {
                    if (!inside(p.credit, 8, p.j, sig_off + sigA_len,
                                pl.regionB * RA2A_SIG_STRIDE_BYTES))
                        return fail(RA2A_EINVAL, "piece credit slot outside region B");
                    if (*u64(p.credit) < p.credit_need)
                        return fail(RA2A_EINVAL, "group %d position %lld: piece %lld waits for a "
                                    "hand-back queued after it (%llu < %llu)", g, (long long)pos,
                                    (long long)idx, (unsigned long long)*u64(p.credit),
                                    (unsigned long long)p.credit_need);
                }
                const int nv = ra2a::plan_vectors(p.pl, V);
                std::vector<std::pair<int64_t, int64_t>> offs;
                rc = walk_plan(p.pl, V, 0, nv, &offs);
                if (rc) return rc;
                for (const auto& o : offs) {
                    const int64_t so = o.first, dofs = o.second;
                    if (!inside(p.src + so, V, p.r, in_off, nb))
                        return fail(RA2A_EINVAL, "piece reads outside in of rank %d", p.r);
                    // the staging is the destination's, or (pull) the sender's own
                    const int stg_rank = pl.pull ? p.r : p.j;
                    if (pl.direct ? !inside(p.dst + dofs, V, p.j, out_off, nb)
                                  : !inside(p.dst + dofs, V, stg_rank, stg_off, pl.ring_bytes))
                        return fail(RA2A_EINVAL, "piece writes outside its destination of rank %d",
                                    pl.direct ? p.j : stg_rank);
                    std::memcpy(&heap[(size_t)(p.dst + dofs)], &heap[(size_t)(p.src + so)],
                                (size_t)V);
                }
                for (int k = 0; k < p.nsig; ++k) {
                    const int64_t sg = p.sig + k * p.sig_step;
                    if (!inside(sg, 8, p.j, sig_off, sigA_len))
                        return fail(RA2A_EINVAL, "piece signal outside region A");
                    if (add)
                        *u64(sg) += 1;
                    else
                        *u64(sg) = 1;
                }
            } else {
                if (idx < 0 || idx >= nitems) return fail(RA2A_EINVAL, "queue item out of range");
                cov_i[(size_t)idx]++;
                const ra2a::Item q = ra2a::item_of(a, g, idx, V);
                if (q.b < 0 || q.b >= a.nbs) return fail(RA2A_EINVAL, "item S-block out of range");
                for (int k = 0; k < q.nsig; ++k) {
                    const int64_t sg = q.sig + k * q.sig_step;
                    if (!inside(sg, 8, q.j, sig_off, sigA_len))
                        return fail(RA2A_EINVAL, "item signal outside region A");
                    if (*u64(sg) != q.sig_want)
                        return fail(RA2A_EINVAL, "group %d position %lld: item %lld waits for "
                                    "pieces queued after it (signal %llu, wants %llu)", g,
                                    (long long)pos, (long long)idx,
                                    (unsigned long long)*u64(sg), (unsigned long long)q.sig_want);
                }
                std::vector<std::pair<int64_t, int64_t>> offs;
                rc = walk_plan(q.pl, V, q.lo, q.hi, &offs);
                if (rc) return rc;
                for (const auto& o : offs) {
                    const int64_t so = o.first, dofs = o.second;
                    const int stg_rank = pl.pull ? q.r0 : q.j;
                    if (!inside(q.src + so, V, stg_rank, stg_off, pl.ring_bytes))
                        return fail(RA2A_EINVAL, "item reads outside the staging of rank %d", stg_rank);
                    if (!inside(q.dst + dofs, V, q.j, out_off, nb))
                        return fail(RA2A_EINVAL, "item writes outside out of rank %d", q.j);
                    std::memcpy(&heap[(size_t)(q.dst + dofs)], &heap[(size_t)(q.src + so)],
                                (size_t)V);
                }
                if (!pl.bulk) {  // the bulk mode has no ring and no hand-back
                    if (!inside(q.credit, 8, q.j, sig_off + sigA_len,
                                pl.regionB * RA2A_SIG_STRIDE_BYTES))
                        return fail(RA2A_EINVAL, "item credit slot outside region B");
                    *u64(q.credit) += 1;
                }
            }
        }
        for (uint8_t x : cov_p)
            if (x != 1) return fail(RA2A_EINVAL, "group %d: queue does not hold every piece once", g);
        for (uint8_t x : cov_i)
            if (x != 1) return fail(RA2A_EINVAL, "group %d: queue does not hold every item once", g);
    }
    for (int j = 0; j < W; ++j) {
        std::memcpy(out[j], &heap[(size_t)(j * stride + out_off)], (size_t)nb);
        if (signals && signals[j])
            for (int64_t k = 0; k < nsig; ++k)
                signals[j][k] = *u64(j * stride + sig_off + k * RA2A_SIG_STRIDE_BYTES);
    }
    return ok();
}
