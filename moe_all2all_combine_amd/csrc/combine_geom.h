// Geometry of the signal-pipelined combine: which bytes each producer piece and
// each consumer work item moves, and which signal slots it touches.  Shared by
// the gfx950 kernel and the host-side plan verifier (compiled for the host), so
// the verifier checks the very index arithmetic the kernel runs.
//
// Combine ("Reverse All2All (EP MoE Distributed Kernel)", section "Reverse
// All2All Operator Semantics"): out_j[s, r*H + h, d] = in_r[j*S + s, h, d].
// Staging of destination j (the page's MTE "Symmetric Memory Layout": a window
// of S-blocks of the output): ring slot `slot` holds rows [0, BS) of
// [H*W][D] columns; source r writes columns r*H + h.
#pragma once

#include <stdint.h>

#include "common.h"

#if defined(__HIPCC__)
#define RA2A_HD __host__ __device__ __forceinline__
#else
#define RA2A_HD inline
#endif

namespace ra2a {

RA2A_HD int64_t geom_min(int64_t a, int64_t b) { return a < b ? a : b; }

// A tile stream: the S-blocks b = 0 .. nbs-1 of destination j, merged head
// block mhb (signal head blocks [hb0, hb0 + nh)), d block db.  Its data moves
// in pieces / units spanning all nh signal tiles at once (their heads are
// adjacent in the input, the staging ring and the output), while each signal
// tile keeps its own signal.
struct Stream {
    int32_t j, mhb, db, hb0, nh;
    int64_t h0, th, d0, td;
};

// Stream sid = (j * nmhb + mhb) * ndb + db.  (32-bit index arithmetic: the
// host keeps every count of tiles, pieces and items below 2^31.)
RA2A_HD Stream stream_of(const PipeArgs& a, int sid) {
    Stream s;
    const uint32_t usid = (uint32_t)sid;
    const uint32_t t = usid / (uint32_t)a.ndb;
    s.db = (int)(usid - t * (uint32_t)a.ndb);
    s.j = (int)(t / (uint32_t)a.nmhb);
    s.mhb = (int)(t - (uint32_t)s.j * (uint32_t)a.nmhb);
    s.hb0 = s.mhb * a.MH;
    s.nh = (int)geom_min(a.MH, a.nhb - s.hb0);
    s.h0 = (int64_t)s.hb0 * a.TH;
    s.th = geom_min((int64_t)s.nh * a.TH, a.H - s.h0);
    s.d0 = (int64_t)s.db * a.TD;
    s.td = geom_min(a.TD, a.D - s.d0);
    return s;
}

// Signal slots of the signal tiles (b, hb0 .. hb0+nh-1, db) (and source r under
// SET): byte offset of the first slot inside slice j's signal array and the
// distance between consecutive head blocks' slots.
RA2A_HD int64_t tile_slot(const PipeArgs& a, int b, int hb, int db, int r) {
    int64_t si = ((int64_t)b * a.nhb + hb) * a.ndb + db;
    return a.protocol == kSigAdd ? si : si * a.W + r;
}
RA2A_HD int64_t slot_step(const PipeArgs& a) {
    return (int64_t)a.ndb * (a.protocol == kSigAdd ? 1 : a.W);
}

// A block of rows: row i (0 <= i < A*B*C) is (ia, ib, ic) and holds `run` bytes
// at src + ia*sa + ib*sb + ic*sc -> dst + ia*da + ib*db + ic*dc.
struct RowPlan {
    int A, B, C;
    int64_t sa, sb, sc;
    int64_t da, db, dc;
    int run;
};

RA2A_HD int plan_vectors(const RowPlan& p, int V) { return p.A * p.B * p.C * (p.run / V); }

// Bytes from a plan's first destination byte to one past its last (the range a
// buffer descriptor for the destination must cover; the host keeps it below 2^32).
RA2A_HD uint32_t plan_span(const RowPlan& p) {
    return (uint32_t)((int64_t)(p.A - 1) * p.da + (int64_t)(p.B - 1) * p.db +
                      (int64_t)(p.C - 1) * p.dc + p.run);
}

// Digits of vector index idx in the plan's mixed radix: idx = ((ia * B + ib) *
// C + ic) * vpr + col, with vpr = run / V vectors per row.
struct PlanDigits {
    int col, ic, ib, ia;
};

RA2A_HD PlanDigits plan_digits(const RowPlan& p, int vpr, uint32_t idx) {
    PlanDigits d;
    const uint32_t row = idx / (uint32_t)vpr;
    d.col = (int)(idx - row * (uint32_t)vpr);
    const uint32_t BC = (uint32_t)p.B * (uint32_t)p.C;
    d.ia = (int)(row / BC);
    const uint32_t rem = row - (uint32_t)d.ia * BC;
    d.ib = (int)(rem / (uint32_t)p.C);
    d.ic = (int)(rem - (uint32_t)d.ib * (uint32_t)p.C);
    return d;
}

// Byte offsets (source, destination) of vector `idx` of a row plan.
RA2A_HD void plan_offsets(const RowPlan& p, int V, int vpr, uint32_t idx, int64_t* so,
                          int64_t* dofs) {
    const PlanDigits d = plan_digits(p, vpr, idx);
    *so = d.ia * p.sa + d.ib * p.sb + d.ic * p.sc + (int64_t)d.col * V;
    *dofs = d.ia * p.da + d.ib * p.db + d.ic * p.dc + (int64_t)d.col * V;
}

// Walks the vectors idx, idx + step, idx + 2 step, ... of a row plan and keeps
// their source / destination offsets with additions and carries only (the
// divisions happen once, in cursor_start).
struct PlanCursor {
    int col, ic, ib;            // digits of the current vector (ia lives in the offsets)
    int scol, sic, sib;         // digits of the step
    int64_t so, dofs;           // offsets of the current vector
    int64_t dso, ddo;           // offsets added by one step before carries
    int64_t cso1, cdo1;         // carry col -> ic
    int64_t cso2, cdo2;         // carry ic -> ib
    int64_t cso3, cdo3;         // carry ib -> ia
};

RA2A_HD PlanCursor cursor_start(const RowPlan& p, int V, int vpr, uint32_t idx, uint32_t step) {
    PlanCursor c;
    const PlanDigits at = plan_digits(p, vpr, idx);
    const PlanDigits st = plan_digits(p, vpr, step);
    c.col = at.col;
    c.ic = at.ic;
    c.ib = at.ib;
    c.scol = st.col;
    c.sic = st.ic;
    c.sib = st.ib;
    c.so = at.ia * p.sa + at.ib * p.sb + at.ic * p.sc + (int64_t)at.col * V;
    c.dofs = at.ia * p.da + at.ib * p.db + at.ic * p.dc + (int64_t)at.col * V;
    c.dso = st.ia * p.sa + st.ib * p.sb + st.ic * p.sc + (int64_t)st.col * V;
    c.ddo = st.ia * p.da + st.ib * p.db + st.ic * p.dc + (int64_t)st.col * V;
    c.cso1 = p.sc - (int64_t)vpr * V;
    c.cdo1 = p.dc - (int64_t)vpr * V;
    c.cso2 = p.sb - p.C * p.sc;
    c.cdo2 = p.db - p.C * p.dc;
    c.cso3 = p.sa - p.B * p.sb;
    c.cdo3 = p.da - p.B * p.db;
    return c;
}

// One step.  Each digit sum is below twice its radix, so one carry per digit suffices.
RA2A_HD void cursor_advance(PlanCursor& c, const RowPlan& p, int vpr) {
    c.so += c.dso;
    c.dofs += c.ddo;
    c.col += c.scol;
    c.ic += c.sic;
    c.ib += c.sib;
    if (c.col >= vpr) {
        c.col -= vpr;
        c.ic += 1;
        c.so += c.cso1;
        c.dofs += c.cdo1;
    }
    if (c.ic >= p.C) {
        c.ic -= p.C;
        c.ib += 1;
        c.so += c.cso2;
        c.dofs += c.cdo2;
    }
    if (c.ib >= p.B) {
        c.ib -= p.B;
        c.so += c.cso3;
        c.dofs += c.cdo3;
    }
}

// Streams of group g: the contiguous range [start, start + ns) of stream ids.
struct GroupStreams {
    int start, ns;
};

// start(g) = floor(g * nstreams / NG), in 32-bit arithmetic: with nstreams =
// q * NG + m, it is g * q + floor(g * m / NG) (g <= NG <= 8, so g * m < 64).
RA2A_HD uint32_t group_start(const PipeArgs& a, uint32_t g) {
    const uint32_t n = (uint32_t)a.nstreams, ng = (uint32_t)a.NG;
    const uint32_t q = n / ng;
    const uint32_t m = n - q * ng;
    return g * q + g * m / ng;
}

RA2A_HD GroupStreams group_streams(const PipeArgs& a, int g) {
    GroupStreams r;
    r.start = (int)group_start(a, (uint32_t)g);
    r.ns = (int)group_start(a, (uint32_t)g + 1u) - r.start;
    return r;
}

// Tile t of a group with ns streams.  Tiles are ordered by stream batch (KB
// consecutive streams), then S-block, then stream inside the batch, so that
// only one batch's staging is live at a time while its S-blocks proceed
// together.  Returns the S-block and the stream's index inside the group.
RA2A_HD void tile_of(const PipeArgs& a, int ns, int64_t t, int* b, int* k) {
    const uint32_t per_batch = (uint32_t)a.nbs * (uint32_t)a.KB;
    const uint32_t ut = (uint32_t)t;
    const uint32_t kb = ut / per_batch;
    const uint32_t rem = ut - kb * per_batch;
    const uint32_t left = (uint32_t)ns - kb * (uint32_t)a.KB;
    const uint32_t nk = left < (uint32_t)a.KB ? left : (uint32_t)a.KB;
    const uint32_t bb = rem / nk;
    *b = (int)bb;
    *k = (int)(kb * (uint32_t)a.KB + (rem - bb * nk));
}

// Producer piece pc of group g: source r = pc mod W of tile pc div W.
struct Piece {
    int32_t b, r, j, slot, nsig;
    int32_t sub, nsub;    // direct mode: the piece's rows are part `sub` of nsub of the tile's
    int64_t cnt;          // direct mode, nsub > 1: the tile's arrival counter (slice j)
    uint64_t cnt_need;    // arrivals that complete the tile (W * nsub under ADD, nsub under SET)
    int64_t src;          // absolute byte offset from the heap base (slice r)
    int64_t dst;          // absolute byte offset (slice j: staging ring, or out if direct)
    RowPlan pl;
    int64_t sig;          // absolute byte offset of its first data signal (slice j)
    int64_t sig_step;     // bytes to the next signal tile's slot
    int64_t credit;       // absolute byte offset of the ring hand-back counter (slice j)
    uint64_t credit_need; // wait until credit >= this (only if b >= R)
    int32_t sid;
    int64_t unit_index;   // first data-signal slot index within slice j (timestamp row)
};

// The piece of source r in S-block b of stream sid: its rows [sub * PR, (sub + 1)
// * PR) of the block (all of them in the staged modes, where PR = BS).
RA2A_HD Piece piece_at(const PipeArgs& a, int sid, int b, int r, int sub = 0) {
    Piece p;
    const int64_t e = a.e;
    p.r = r;
    p.b = b;
    p.sid = sid;
    p.sub = sub;
    const Stream st = stream_of(a, p.sid);
    p.j = st.j;
    const uint32_t cycle = (uint32_t)p.b / (uint32_t)a.R;  // uses of this ring slot before b
    p.slot = (int)((uint32_t)p.b - cycle * (uint32_t)a.R);
    const bool add = a.protocol == kSigAdd;
    const int64_t HWDe = a.H * (int64_t)a.W * a.D * e;
    const int64_t blk = geom_min(a.BS, a.S - (int64_t)p.b * a.BS);  // rows of the block
    p.nsub = (int)((blk + a.PR - 1) / a.PR);
    const int64_t s0 = (int64_t)p.b * a.BS + (int64_t)sub * a.PR;
    const int bs = (int)geom_min(a.PR, blk - (int64_t)sub * a.PR);
    RowPlan& pl = p.pl;
    pl.A = bs;
    if (a.inverse) {
        // dispatch: source rank p.r sends in_r[s0.., j*H + h0.., d0..] (rows of
        // [H*W][D] columns) to out_j[r*S + s0.., h0.., d0..] (rows of [H][D])
        p.src = (int64_t)p.r * a.stride + a.in_off + s0 * HWDe + ((int64_t)st.j * a.H + st.h0) * a.D * e +
                st.d0 * e;
        p.dst = (int64_t)st.j * a.stride + a.out_off +
                (((int64_t)p.r * a.S + s0) * a.H + st.h0) * a.D * e + st.d0 * e;
        pl.sa = HWDe;
        pl.da = a.H * a.D * e;
    } else if (a.bulk) {
        // bulk staging of destination j: sender r's segment in the input's own
        // layout, [r][s][h][d], so both sides have rows of H*D elements.  Pull:
        // the sender's own staging [j][s][h][d] in slice r, the same bytes at the
        // same offset as its input rows for j (a local copy)
        p.src = (int64_t)p.r * a.stride + a.in_off + (((int64_t)st.j * a.S + s0) * a.H + st.h0) * a.D * e +
                st.d0 * e;
        p.dst = a.pull ? (int64_t)p.r * a.stride + a.stg_off +
                             (((int64_t)st.j * a.S + s0) * a.H + st.h0) * a.D * e + st.d0 * e
                       : (int64_t)st.j * a.stride + a.stg_off +
                             (((int64_t)p.r * a.S + s0) * a.H + st.h0) * a.D * e + st.d0 * e;
        pl.sa = pl.da = a.H * a.D * e;
    } else {
        p.src = (int64_t)p.r * a.stride + a.in_off + (((int64_t)st.j * a.S + s0) * a.H + st.h0) * a.D * e +
                st.d0 * e;
        // staging ring slot, or (direct) the piece's final place in out_j: both are
        // rows of [H*W][D] columns, the ring being a window of S-blocks of the output
        p.dst = a.direct ? (int64_t)st.j * a.stride + a.out_off + s0 * HWDe
                         : (int64_t)st.j * a.stride + a.stg_off + (int64_t)p.slot * a.BS * HWDe;
        p.dst += ((int64_t)p.r * a.H + st.h0) * a.D * e + st.d0 * e;
        pl.sa = a.H * a.D * e;  // input token stride
        pl.da = HWDe;           // staging token stride
    }
    pl.C = 1;
    pl.sc = pl.dc = 0;
    if (st.td == a.D) {     // the tile spans D: its heads form one run
        pl.B = 1;
        pl.sb = pl.db = 0;
        pl.run = (int)(st.th * a.D * e);
    } else {
        pl.B = (int)st.th;
        pl.sb = pl.db = a.D * e;
        pl.run = (int)(st.td * e);
    }
    const int64_t sig_base = (int64_t)st.j * a.stride + a.sig_off;
    p.nsig = st.nh;
    p.unit_index = tile_slot(a, p.b, st.hb0, st.db, p.r);
    p.sig = sig_base + p.unit_index * kSigStrideU64 * 8;
    p.sig_step = slot_step(a) * kSigStrideU64 * 8;
    int64_t ci = ((int64_t)p.slot * a.nmhb + st.mhb) * a.ndb + st.db;
    if (!add) ci = ci * a.W + p.r;
    p.credit = sig_base + (a.regionA + ci) * kSigStrideU64 * 8;
    p.credit_need = (uint64_t)cycle * (uint64_t)a.csplit;
    // direct mode with several pieces per tile and source: one arrival counter per
    // moved tile (b, merged head block, d block) -- per source under SET -- in region B
    int64_t ti = ((int64_t)p.b * a.nmhb + st.mhb) * a.ndb + st.db;
    if (!add) ti = ti * a.W + p.r;
    p.cnt = sig_base + (a.regionA + ti) * kSigStrideU64 * 8;
    p.cnt_need = (uint64_t)p.nsub * (add ? (uint64_t)a.W : 1ull);
    return p;
}

// Staged mode: producer piece pc of group g, source r = pc mod W of the
// group's tile pc div W (tile_of order).
RA2A_HD Piece piece_of(const PipeArgs& a, int g, int64_t pc) {
    const GroupStreams gs = group_streams(a, g);
    const uint32_t tile = (uint32_t)pc / (uint32_t)a.W;
    const int r = (int)((uint32_t)pc - tile * (uint32_t)a.W);
    int b, k;
    tile_of(a, gs.ns, tile, &b, &k);
    return piece_at(a, gs.start + k, b, r);
}

RA2A_HD int64_t group_pieces(const PipeArgs& a, int g) {
    return (int64_t)a.nbs * group_streams(a, g).ns * a.W;
}

// Direct mode: pieces per source in one stream: nsub for every S-block but the
// last, which has ceil(its rows / PR).
RA2A_HD int64_t stream_subtiles(const PipeArgs& a) {
    const int64_t last = a.S - (int64_t)(a.nbs - 1) * a.BS;
    return (int64_t)(a.nbs - 1) * a.nsub + (last + a.PR - 1) / a.PR;
}

// Direct mode: piece gp of the whole combine, in the order (stream, S-block,
// part, source) with the source fastest, so that the pieces in flight together
// fill a few destinations' outputs and read contiguous row ranges of every input.
RA2A_HD Piece direct_piece(const PipeArgs& a, int64_t gp) {
    const uint32_t t = (uint32_t)gp / (uint32_t)a.W;
    const int r = (int)((uint32_t)gp - t * (uint32_t)a.W);
    const uint32_t spt = (uint32_t)stream_subtiles(a);
    const uint32_t sid = t / spt;
    const uint32_t rem = t - sid * spt;
    uint32_t b = rem / (uint32_t)a.nsub;
    if (b > (uint32_t)a.nbs - 1u) b = (uint32_t)a.nbs - 1u;  // the last block may be short
    return piece_at(a, (int)sid, (int)b, r, (int)(rem - b * (uint32_t)a.nsub));
}

RA2A_HD int64_t total_pieces(const PipeArgs& a) {
    return stream_subtiles(a) * a.nstreams * a.W;
}

// Row units (direct mode).  A combine row unit fills rows [s0, s0 + rows) of
// out_j completely: for each of those tokens the W sources' runs of H*D
// elements, which are contiguous in out_j (columns r*H .. r*H + H - 1 for
// r = 0 .. W-1 make up a whole output row) and contiguous, token after token, in
// each in_r (rows j*S + s0 ..).  So a unit writes one contiguous range of out_j
// and reads W contiguous ranges.  It copies source by source (one source's rows,
// then the next source's): on gfx950 reading each range in order while the
// output fills as W interleaved streams measured faster than filling the output
// token by token (W = 8, S = 512, H = 16, D = 128 bf16: 47 against 60 us).
// The dispatch's row unit is the mirror image: source j's rows [s0, s0 + rows)
// of in_j, read whole, give each destination r one contiguous range, rows
// j*S + s0 .. of out_r, destination by destination.
// The signal tiles of S-block b are complete once every unit of b has stored
// its rows: each unit releases its stores device-wide and adds 1 to the block's
// arrival counter (region B of slice j); the unit that brings it to `nub` (the
// block's unit count) marks every signal tile of the block complete -- ADD W on
// the tile's slot, or SET 1 on each (tile, source) slot (the dispatch: in every
// destination's slice) -- exactly the values W pieces would have left; or, under
// ADD with nub dividing W, every unit adds W / nub itself (the kernel's choice).
// Units are ordered S-block first, then the unit inside the block, then j, so
// that early tiles of every destination complete first.
struct RowUnit {
    int32_t j, b, k, rows, nub;
    int64_t src;          // absolute byte offset of in_0[j*S + s0] (slice 0); source r is
                          // r slices further (the plan's middle digit)
    int64_t dst;          // absolute byte offset of out_j[s0] (slice j)
    RowPlan pl;
    int64_t sig;          // absolute byte offset of the block's first data signal (slice j;
                          // the dispatch: in destination slice 0)
    int32_t nsig;         // data-signal slots of the block, per destination
    int64_t sig_step;     // bytes between consecutive ones
    int32_t nd;           // destinations signalled: 1 (the combine: j) or W (the dispatch)
    int64_t unit_index;   // slot index of the block's first data signal (timestamp row)
    int64_t unit_step;    // slot distance between consecutive ones
    int64_t cnt;          // absolute byte offset of the block's arrival counter (slice j)
};

// Row units of S-block b (of any destination).
RA2A_HD int32_t row_units_of_block(const PipeArgs& a, int b) {
    const int64_t bs = geom_min(a.BS, a.S - (int64_t)b * a.BS);
    return (int32_t)((bs + a.KU - 1) / a.KU);
}

RA2A_HD int64_t total_row_units(const PipeArgs& a) {
    return ((int64_t)(a.nbs - 1) * a.upb + row_units_of_block(a, a.nbs - 1)) * a.W;
}

RA2A_HD RowUnit row_unit(const PipeArgs& a, int64_t u) {
    RowUnit q;
    const int64_t e = a.e;
    const uint32_t per_block = (uint32_t)a.upb * (uint32_t)a.W;  // units of a full S-block
    uint32_t b = (uint32_t)u / per_block;
    if (b > (uint32_t)a.nbs - 1u) b = (uint32_t)a.nbs - 1u;      // the last block may be short
    const uint32_t rem = (uint32_t)u - b * per_block;
    const uint32_t k = rem / (uint32_t)a.W;
    q.b = (int)b;
    q.k = (int)k;
    q.j = (int)(rem - k * (uint32_t)a.W);
    q.nub = row_units_of_block(a, q.b);
    const int64_t bs = geom_min(a.BS, a.S - (int64_t)q.b * a.BS);
    const int64_t s0 = (int64_t)q.b * a.BS + (int64_t)q.k * a.KU;
    q.rows = (int)geom_min(a.KU, bs - (int64_t)q.k * a.KU);
    const int64_t run = a.H * a.D * e;  // one source's part of a token row
    RowPlan& pl = q.pl;
    const int64_t sig_j = (int64_t)q.j * a.stride + a.sig_off;
    q.cnt = sig_j + (a.regionA + q.b) * kSigStrideU64 * 8;
    if (a.inverse) {
        // the dispatch: unit (source j, rows s0 ..) reads whole rows of in_j
        // ([H*W][D] columns) and gives each destination r its run, rows j*S + s0 ..
        // of out_r: destination by destination, each one contiguous range
        q.src = (int64_t)q.j * a.stride + a.in_off + s0 * run * a.W;
        q.dst = a.out_off + ((int64_t)q.j * a.S + s0) * run;  // destination r: r slices further
        pl.A = a.W;       // destinations
        pl.sa = run;
        pl.da = a.stride;
        pl.B = q.rows;    // tokens
        pl.sb = run * a.W;
        pl.db = run;
        pl.C = 1;
        pl.sc = pl.dc = 0;
        pl.run = (int)run;
        // SET per (tile, source j) in each destination's slice
        q.unit_index = tile_slot(a, q.b, 0, 0, q.j);
        q.unit_step = a.W;
        q.sig = a.sig_off + q.unit_index * kSigStrideU64 * 8;
        q.nsig = a.nhb * a.ndb;
        q.sig_step = (int64_t)a.W * kSigStrideU64 * 8;
        q.nd = a.W;
        return q;
    }
    q.src = a.in_off + ((int64_t)q.j * a.S + s0) * run;
    q.dst = (int64_t)q.j * a.stride + a.out_off + s0 * run * a.W;
    pl.A = a.W;         // sources: each one's rows are read in one contiguous range
    pl.sa = a.stride;
    pl.da = run;
    pl.B = q.rows;      // tokens
    pl.sb = run;
    pl.db = run * a.W;
    pl.C = 1;
    pl.sc = pl.dc = 0;
    pl.run = (int)run;
    const int64_t per_block_slots = (int64_t)a.nhb * a.ndb * (a.protocol == kSigAdd ? 1 : a.W);
    q.unit_index = (int64_t)q.b * per_block_slots;
    q.unit_step = 1;
    q.sig = sig_j + q.unit_index * kSigStrideU64 * 8;
    q.nsig = (int32_t)per_block_slots;
    q.sig_step = kSigStrideU64 * 8;
    q.nd = 1;
    return q;
}

// Consumer work item `it` of group g: part `part` of a unit (ADD: a tile with
// all W sources; SET: one source of a tile, units ordered tile then source),
// i.e. the unit's vectors [lo, hi) of its row plan.  A unit spans the nsig
// signal tiles of its stream and may start once every one of them is complete.
struct Item {
    int32_t b, j, r0, nsrc, slot, part, nsig;
    int64_t src;          // absolute byte offset (slice j, staging ring)
    int64_t dst;          // absolute byte offset (slice j, out)
    RowPlan pl;
    int lo, hi;
    int64_t sig;          // first data signal to wait on
    int64_t sig_step;     // bytes to the next signal tile's slot
    uint64_t sig_want;    // W (ADD) or 1 (SET)
    int64_t credit;       // hand-back counter to add 1 to
    int64_t unit_index;   // first data-signal slot index within slice j (timestamp row)
    int64_t unit_step;    // slot-index distance to the next signal tile
};

RA2A_HD Item item_of(const PipeArgs& a, int g, int64_t it, int V) {
    Item q;
    const int64_t e = a.e;
    const bool add = a.protocol == kSigAdd;
    const GroupStreams gs = group_streams(a, g);
    const uint32_t u = (uint32_t)it / (uint32_t)a.csplit;
    q.part = (int)((uint32_t)it - u * (uint32_t)a.csplit);
    const uint32_t t = add ? u : u / (uint32_t)a.W;
    q.r0 = add ? 0 : (int)(u - t * (uint32_t)a.W);
    q.nsrc = add ? a.W : 1;
    int k;
    tile_of(a, gs.ns, t, &q.b, &k);
    const Stream st = stream_of(a, gs.start + k);
    q.j = st.j;
    q.slot = (int)((uint32_t)q.b % (uint32_t)a.R);
    const int64_t HWDe = a.H * (int64_t)a.W * a.D * e;
    const int64_t s0 = (int64_t)q.b * a.BS;
    const int bs = (int)geom_min(a.BS, a.S - s0);
    const int64_t col = ((int64_t)q.r0 * a.H + st.h0) * a.D * e + st.d0 * e;
    // the ring holds rows of the output's layout; the bulk staging (one source
    // per unit, the SET layout) holds sender r0's rows of H*D elements, in slice
    // j at [r0][s][h][d], or (pull) in sender r0's own slice at [j][s][h][d]
    q.src = a.pull   ? (int64_t)q.r0 * a.stride + a.stg_off +
                         (((int64_t)st.j * a.S + s0) * a.H + st.h0) * a.D * e + st.d0 * e
            : a.bulk ? (int64_t)st.j * a.stride + a.stg_off +
                         (((int64_t)q.r0 * a.S + s0) * a.H + st.h0) * a.D * e + st.d0 * e
                     : (int64_t)st.j * a.stride + a.stg_off + (int64_t)q.slot * a.BS * HWDe + col;
    q.dst = (int64_t)st.j * a.stride + a.out_off + s0 * HWDe + col;
    RowPlan& pl = q.pl;
    const int64_t head = a.D * e;
    pl.A = bs;
    pl.sa = a.bulk ? a.H * head : HWDe;
    pl.da = HWDe;
    if (st.td == a.D && st.th == a.H) {  // whole rows of the sources: one run
        pl.B = 1;
        pl.C = 1;
        pl.sb = pl.db = pl.sc = pl.dc = 0;
        pl.run = (int)(q.nsrc * a.H * a.D * e);
    } else if (st.td == a.D) {  // heads of one source merge
        pl.B = q.nsrc;
        pl.sb = pl.db = a.H * head;
        pl.C = 1;
        pl.sc = pl.dc = 0;
        pl.run = (int)(st.th * a.D * e);
    } else {
        pl.B = q.nsrc;
        pl.sb = pl.db = a.H * head;
        pl.C = (int)st.th;
        pl.sc = pl.dc = head;
        pl.run = (int)(st.td * e);
    }
    // part p of the unit's nvec vectors: [floor(nvec p / cs), floor(nvec (p+1) / cs)),
    // in 32-bit arithmetic with nvec = qv * cs + mv
    const uint32_t nvec = (uint32_t)plan_vectors(pl, V);
    const uint32_t cs = (uint32_t)a.csplit, up = (uint32_t)q.part;
    const uint32_t qv = nvec / cs, mv = nvec - qv * cs;
    q.lo = (int)(up * qv + up * mv / cs);
    q.hi = (int)((up + 1u) * qv + (up + 1u) * mv / cs);
    const int64_t sig_base = (int64_t)st.j * a.stride + a.sig_off;
    q.nsig = st.nh;
    q.unit_index = tile_slot(a, q.b, st.hb0, st.db, q.r0);
    q.unit_step = slot_step(a);
    q.sig = sig_base + q.unit_index * kSigStrideU64 * 8;
    q.sig_step = q.unit_step * kSigStrideU64 * 8;
    q.sig_want = add ? (uint64_t)a.W : 1ull;
    int64_t ci = ((int64_t)q.slot * a.nmhb + st.mhb) * a.ndb + st.db;
    if (!add) ci = ci * a.W + q.r0;
    q.credit = sig_base + (a.regionA + ci) * kSigStrideU64 * 8;
    return q;
}

RA2A_HD int64_t group_items(const PipeArgs& a, int g) {
    const bool add = a.protocol == kSigAdd;
    return (int64_t)a.nbs * group_streams(a, g).ns * (add ? 1 : a.W) * a.csplit;
}

// The work queue of group g.  Its tasks are the group's producer pieces and
// consumer work items in one order in which every wait of a task is on a task
// placed before it: the pieces of tile t + L, then the consumer items of tile
// t, for t = 0, 1, ... (after the pieces of tiles 0 .. L-1).  A piece of tile
// (k, b) waits for the hand-back of tile (k, b - R), which lies R * nk tiles
// earlier in the same stream batch (nk streams), so L <= R * nk - 1 keeps that
// dependency backwards; without ring reuse nothing waits on consumers and any
// L is valid.  Workgroups claim tasks in queue order
// and only ever wait on earlier tasks, each of which a running workgroup has
// claimed; hence no deadlock, whatever the number of resident workgroups.
struct GroupQueue {
    int64_t ntiles;  // tiles of the group
    int np, ni;      // pieces per tile (W), consumer items per tile
    int64_t L;       // lookahead in tiles
    int64_t total;   // tasks
};

RA2A_HD GroupQueue group_queue(const PipeArgs& a, int g) {
    GroupQueue q;
    const int ns = group_streams(a, g).ns;
    q.ntiles = (int64_t)a.nbs * ns;
    q.np = a.W;
    q.ni = (a.protocol == kSigAdd ? 1 : a.W) * a.csplit;
    if (a.direct || ns == 0) {
        q.L = q.ntiles;
    } else {
        // smallest stream batch of the group (the last one may be partial)
        const int nk_last = ns - ((ns - 1) / a.KB) * a.KB;
        const int nk_min = nk_last < a.KB ? nk_last : a.KB;
        const int64_t cap = (int64_t)a.R * nk_min - 1;
        // default: half the run-ahead the ring allows, so that a piece's hand-back
        // and a unit's pieces were both claimed well before they are needed
        if (a.lookahead < 0 || (a.lookahead == 0 && a.R >= a.nbs))
            q.L = q.ntiles;  // (no ring reuse: nothing waits on consumers)
        else
            q.L = a.lookahead > 0 ? a.lookahead : (cap + 1) / 2 > 1 ? (cap + 1) / 2 : 1;
        if (a.R < a.nbs && q.L > cap) q.L = cap;  // ring reused: no wait may point forward
        if (q.L > q.ntiles) q.L = q.ntiles;
    }
    q.total = q.ntiles * (q.np + q.ni);
    return q;
}

// Task at queue position pos: returns true for a piece (index *idx into the
// group's pieces) or false for a consumer item (index *idx into its items).
RA2A_HD bool task_of(const GroupQueue& q, int64_t pos, int64_t* idx) {
    const int64_t head = q.L * q.np;
    if (pos < head) {
        *idx = pos;
        return true;
    }
    pos -= head;
    const int64_t blk = q.np + q.ni;
    const int64_t nfull = q.ntiles - q.L;  // blocks: pieces of tile t+L, items of tile t
    if (pos < nfull * blk) {
        const int64_t t = (uint32_t)pos / (uint32_t)blk;  // positions < 2^31
        const int64_t off = pos - t * blk;
        if (off < q.np) {
            *idx = (t + q.L) * q.np + off;
            return true;
        }
        *idx = t * q.ni + (off - q.np);
        return false;
    }
    pos -= nfull * blk;
    *idx = nfull * q.ni + pos;  // items of the last L tiles
    return false;
}

}  // namespace ra2a
