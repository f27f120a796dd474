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

struct Stream {
    int32_t j, hb, db;
    int64_t h0, th, d0, td;
};

// Stream sid = (j * nhb + hb) * ndb + db: destination j, head block hb, d block db.
RA2A_HD Stream stream_of(const PipeArgs& a, int sid) {
    Stream s;
    s.db = sid % a.ndb;
    const int t = sid / a.ndb;
    s.hb = t % a.nhb;
    s.j = t / a.nhb;
    s.h0 = (int64_t)s.hb * a.TH;
    s.th = geom_min(a.TH, a.H - s.h0);
    s.d0 = (int64_t)s.db * a.TD;
    s.td = geom_min(a.TD, a.D - s.d0);
    return s;
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

// Byte offsets (source, destination) of vector `idx` of a row plan.
RA2A_HD void plan_offsets(const RowPlan& p, int V, int vpr, int BC, int idx, int64_t* so,
                          int64_t* dofs) {
    const int row = idx / vpr;
    const int col = idx - row * vpr;
    const int ia = row / BC;
    const int rem = row - ia * BC;
    const int ib = rem / p.C;
    const int ic = rem - ib * p.C;
    *so = ia * p.sa + ib * p.sb + ic * p.sc + (int64_t)col * V;
    *dofs = ia * p.da + ib * p.db + ic * p.dc + (int64_t)col * V;
}

// Streams of group g: the contiguous range [start, start + ns) of stream ids.
struct GroupStreams {
    int start, ns;
};

RA2A_HD GroupStreams group_streams(const PipeArgs& a, int g) {
    GroupStreams r;
    r.start = (int)((int64_t)g * a.nstreams / a.NG);
    r.ns = (int)((int64_t)(g + 1) * a.nstreams / a.NG) - r.start;
    return r;
}

// Tile t of a group with ns streams.  Tiles are ordered by stream batch (KB
// consecutive streams), then S-block, then stream inside the batch, so that
// only one batch's staging is live at a time while its S-blocks proceed
// together.  Returns the S-block and the stream's index inside the group.
RA2A_HD void tile_of(const PipeArgs& a, int ns, int64_t t, int* b, int* k) {
    const int64_t per_batch = (int64_t)a.nbs * a.KB;
    const int kb = (int)(t / per_batch);
    const int64_t rem = t - kb * per_batch;
    const int left = ns - kb * a.KB;
    const int nk = left < a.KB ? left : a.KB;
    *b = (int)(rem / nk);
    *k = kb * a.KB + (int)(rem - (int64_t)(*b) * nk);
}

// Producer piece pc of group g: source r = pc mod W of tile pc div W.
struct Piece {
    int32_t b, r, j, slot;
    int64_t src;          // absolute byte offset from the heap base (slice r)
    int64_t dst;          // absolute byte offset (slice j, staging ring)
    RowPlan pl;
    int64_t sig;          // absolute byte offset of its data signal (slice j)
    int64_t credit;       // absolute byte offset of the ring hand-back counter (slice j)
    uint64_t credit_need; // wait until credit >= this (only if b >= R)
    int32_t sid;
};

RA2A_HD Piece piece_of(const PipeArgs& a, int g, int64_t pc) {
    Piece p;
    const int64_t e = a.e;
    const GroupStreams gs = group_streams(a, g);
    p.r = (int)(pc % a.W);
    int k;
    tile_of(a, gs.ns, pc / a.W, &p.b, &k);
    p.sid = gs.start + k;
    const Stream st = stream_of(a, p.sid);
    p.j = st.j;
    p.slot = p.b % a.R;
    const bool add = a.protocol == kSigAdd;
    const int64_t HWDe = a.H * (int64_t)a.W * a.D * e;
    const int64_t s0 = (int64_t)p.b * a.BS;
    const int bs = (int)geom_min(a.BS, a.S - s0);
    p.src = (int64_t)p.r * a.stride + a.in_off + (((int64_t)st.j * a.S + s0) * a.H + st.h0) * a.D * e +
            st.d0 * e;
    p.dst = (int64_t)st.j * a.stride + a.stg_off + (int64_t)p.slot * a.BS * HWDe +
            ((int64_t)p.r * a.H + st.h0) * a.D * e + st.d0 * e;
    RowPlan& pl = p.pl;
    pl.A = bs;
    pl.sa = a.H * a.D * e;  // input token stride
    pl.da = HWDe;           // staging token stride
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
    int64_t si = ((int64_t)p.b * a.nhb + st.hb) * a.ndb + st.db;
    if (!add) si = si * a.W + p.r;
    p.sig = (int64_t)st.j * a.stride + a.sig_off + si * kSigStrideU64 * 8;
    int64_t ci = ((int64_t)p.slot * a.nhb + st.hb) * a.ndb + st.db;
    if (!add) ci = ci * a.W + p.r;
    p.credit = (int64_t)st.j * a.stride + a.sig_off + (a.regionA + ci) * kSigStrideU64 * 8;
    p.credit_need = (uint64_t)(p.b / a.R) * (uint64_t)a.csplit;
    return p;
}

RA2A_HD int64_t group_pieces(const PipeArgs& a, int g) {
    return (int64_t)a.nbs * group_streams(a, g).ns * a.W;
}

// Consumer work item `it` of group g: part `part` of a unit (ADD: a tile with
// all W sources; SET: one source of a tile, units ordered tile then source),
// i.e. the unit's vectors [lo, hi) of its row plan.
struct Item {
    int32_t b, j, r0, nsrc, slot, part;
    int64_t src;          // absolute byte offset (slice j, staging ring)
    int64_t dst;          // absolute byte offset (slice j, out)
    RowPlan pl;
    int lo, hi;
    int64_t sig;          // data signal to wait on
    uint64_t sig_want;    // W (ADD) or 1 (SET)
    int64_t credit;       // hand-back counter to add 1 to
    int64_t unit_index;   // data-signal slot index within slice j (timestamp row)
};

RA2A_HD Item item_of(const PipeArgs& a, int g, int64_t it, int V) {
    Item q;
    const int64_t e = a.e;
    const bool add = a.protocol == kSigAdd;
    const GroupStreams gs = group_streams(a, g);
    q.part = (int)(it % a.csplit);
    const int64_t u = it / a.csplit;
    const int64_t t = add ? u : u / a.W;
    q.r0 = add ? 0 : (int)(u % a.W);
    q.nsrc = add ? a.W : 1;
    int k;
    tile_of(a, gs.ns, t, &q.b, &k);
    const Stream st = stream_of(a, gs.start + k);
    q.j = st.j;
    q.slot = q.b % a.R;
    const int64_t HWDe = a.H * (int64_t)a.W * a.D * e;
    const int64_t s0 = (int64_t)q.b * a.BS;
    const int bs = (int)geom_min(a.BS, a.S - s0);
    const int64_t col = ((int64_t)q.r0 * a.H + st.h0) * a.D * e + st.d0 * e;
    q.src = (int64_t)st.j * a.stride + a.stg_off + (int64_t)q.slot * a.BS * HWDe + col;
    q.dst = (int64_t)st.j * a.stride + a.out_off + s0 * HWDe + col;
    RowPlan& pl = q.pl;
    const int64_t head = a.D * e;
    pl.A = bs;
    pl.sa = pl.da = HWDe;
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
    const int nvec = plan_vectors(pl, V);
    q.lo = (int)((int64_t)nvec * q.part / a.csplit);
    q.hi = (int)((int64_t)nvec * (q.part + 1) / a.csplit);
    int64_t si = ((int64_t)q.b * a.nhb + st.hb) * a.ndb + st.db;
    if (!add) si = si * a.W + q.r0;
    q.unit_index = si;
    q.sig = (int64_t)st.j * a.stride + a.sig_off + si * kSigStrideU64 * 8;
    q.sig_want = add ? (uint64_t)a.W : 1ull;
    int64_t ci = ((int64_t)q.slot * a.nhb + st.hb) * a.ndb + st.db;
    if (!add) ci = ci * a.W + q.r0;
    q.credit = (int64_t)st.j * a.stride + a.sig_off + (a.regionA + ci) * kSigStrideU64 * 8;
    return q;
}

RA2A_HD int64_t group_items(const PipeArgs& a, int g) {
    const bool add = a.protocol == kSigAdd;
    return (int64_t)a.nbs * group_streams(a, g).ns * (add ? 1 : a.W) * a.csplit;
}

// Role of workgroup `wg` of the persistent grid.
struct Role {
    int g;          // stream group
    bool producer;
    int index;      // producer index or consumer index inside the group
};

RA2A_HD Role role_of(const PipeArgs& a, int wg) {
    Role r;
    r.g = wg % a.NG;
    const int lg = wg / a.NG;
    const int per = lg / a.q;
    const int pos = lg - per * a.q;
    r.producer = pos < a.p;
    r.index = r.producer ? per * a.p + pos : per * (a.q - a.p) + (pos - a.p);
    return r;
}

}  // namespace ra2a
