"""Expected final signal arrays of one slice, laid out as the combine lays them
out (data signals, then ring hand-back counters; the work-queue words that
follow are not part of the protocol), from the protocol model's closed forms in
``oracle.protocol``."""
import math

import numpy as np

import moe_all2all_combine_amd as ra2a
from oracle.protocol import (ADD, SET, ProtocolSpec, expected_final_block_counts,
                             expected_final_credits, expected_final_piece_counts,
                             expected_final_signals)

ELEM = {"u8": 1, "bf16": 2, "f16": 2, "i32": 4, "f32": 4, "i64": 8, "f64": 8}


def row_mode(W, S, H, D, opts, dtype="bf16") -> bool:
    """Whether the combine resolves these options to row units (asked for, or
    mode 0 on a shape whose default is row units): the plan the library reports."""
    return ra2a.rev_all2all_plan(W, S, H, D, dtype, opts).mode == ra2a.MODE_ROWS


def unit_rows(W, S, H, D, opts, dtype="bf16") -> int:
    """Tokens per row unit as the header documents it."""
    tile_s = min(opts.tile_s or min(S, 64), S)
    row = W * H * D * ELEM[dtype]
    ku = min(opts.unit_rows or max(1, 262144 // row), tile_s)
    if not opts.unit_rows and H * D * ELEM[dtype] >= 4096:
        ku2 = min(max(1, 524288 // row), tile_s)
        nbs = math.ceil(S / tile_s)
        units2 = ((nbs - 1) * math.ceil(tile_s / ku2) + math.ceil((S - (nbs - 1) * tile_s) / ku2)) * W
        if units2 >= 256:
            ku = ku2
    return ku


def expected_signal_array(W, S, H, D, opts, csplit, dtype="bf16"):
    """Data signals (one per signal tile) then hand-back counters (one per ring
    slot of each moved stream, a stream being head_merge adjacent head blocks),
    or, with row units, one arrival counter per S-block."""
    tile_s = opts.tile_s or min(S, 64)
    nbs = math.ceil(S / tile_s)
    nhb = math.ceil(H / (opts.tile_h or 1))
    ndb = math.ceil(D / (opts.tile_d or D))
    direct = opts.mode not in (ra2a.MODE_STAGED, ra2a.MODE_BULK, ra2a.MODE_PULL)
    bulk = opts.mode in (ra2a.MODE_BULK, ra2a.MODE_PULL)  # staged, but no ring: data signals only
    R = nbs if (direct or bulk) else min(opts.ring or 8, nbs)
    if direct:
        csplit = 1
    # the dispatch fills each tile from one source: one slot per (tile, source), SET 1
    dispatch = getattr(opts, "direction", 0) == ra2a.DIR_DISPATCH
    proto = SET if (opts.protocol == ra2a.PROTO_SET or dispatch or bulk) else ADD
    per = W if proto == SET else 1
    # merged head blocks: derived from the size of the hand-back region
    _, n_credit, _ = ra2a.rev_all2all_signal_slots(W, S, H, D, dtype, opts)
    if row_mode(W, S, H, D, opts, dtype):
        tiles = ProtocolSpec(W=W, nbs=nbs, nstreams=nhb * ndb, R=R, protocol=proto)
        ns = nhb * ndb
        a = np.zeros(nbs * ns * per, dtype=np.int64)
        for k, v in expected_final_signals(tiles).items():
            if k[0] == 0:
                a[(k[2] * ns + k[1]) * per + (k[3] if proto == SET else 0)] = v
        b = np.asarray(expected_final_block_counts(S, tile_s, unit_rows(W, S, H, D, opts, dtype)),
                       dtype=np.int64)
        assert n_credit == nbs
        return np.concatenate([a, b])
    if direct or bulk:
        # no ring (direct: no consumer work either): the data signals, then (direct
        # mode with tiles cut into several pieces) one arrival counter per moved tile
        tiles = ProtocolSpec(W=W, nbs=nbs, nstreams=nhb * ndb, R=R, protocol=proto)
        ns = nhb * ndb
        a = np.zeros(nbs * ns * per, dtype=np.int64)
        for k, v in expected_final_signals(tiles).items():
            if k[0] == 0:
                a[(k[2] * ns + k[1]) * per + (k[3] if proto == SET else 0)] = v
        plan = ra2a.rev_all2all_plan(W, S, H, D, dtype, opts) if direct else None
        if plan is None or plan.pieces_per_tile == 1:
            assert n_credit == 0
            return a
        nm = n_credit // (nbs * per)  # moved tiles per S-block: merged head blocks x d blocks
        assert nm * nbs * per == n_credit
        cnt = expected_final_piece_counts(S, tile_s, plan.piece_rows, W, proto)
        b = np.repeat(np.asarray(cnt, dtype=np.int64), nm * per)
        return np.concatenate([a, b])
    nmhb = n_credit // (R * ndb * per)
    assert nmhb * R * ndb * per == n_credit
    # data signals: one per signal tile, the model's closed form
    tiles = ProtocolSpec(W=W, nbs=nbs, nstreams=nhb * ndb, R=R, protocol=proto)
    ns = nhb * ndb
    a = np.zeros(nbs * ns * per, dtype=np.int64)
    for k, v in expected_final_signals(tiles).items():
        if k[0] != 0:
            continue
        a[(k[2] * ns + k[1]) * per + (k[3] if proto == SET else 0)] = v
    # hand-back counters: one per (ring slot, moved stream), the model's closed form
    moved = ProtocolSpec(W=W, nbs=nbs, nstreams=nmhb * ndb, R=R, protocol=proto)
    nm = nmhb * ndb
    b = np.zeros(R * nm * per, dtype=np.int64)
    for k, v in expected_final_credits(moved).items():
        if k[0] != 0:
            continue
        b[(k[2] * nm + k[1]) * per + (k[3] if proto == SET else 0)] = v * csplit
    return np.concatenate([a, b])
