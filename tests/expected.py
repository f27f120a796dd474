"""Expected final signal arrays of one slice, laid out as the combine lays them
out (data signals, then ring hand-back counters), from the protocol model's
closed forms in ``oracle.protocol``."""
import math

import numpy as np

import moe_all2all_combine_amd as ra2a
from oracle.protocol import ADD, SET, ProtocolSpec, expected_final_credits, expected_final_signals


def expected_signal_array(W, S, H, D, opts, csplit):
    nbs = math.ceil(S / opts.tile_s)
    nhb = math.ceil(H / opts.tile_h)
    ndb = math.ceil(D / opts.tile_d)
    R = min(opts.ring or 2, nbs)
    proto = SET if opts.protocol == ra2a.PROTO_SET else ADD
    spec = ProtocolSpec(W=W, nbs=nbs, nstreams=nhb * ndb, R=R, protocol=proto)
    ns = nhb * ndb
    per = W if proto == SET else 1
    a = np.zeros(nbs * ns * per, dtype=np.int64)
    for k, v in expected_final_signals(spec).items():
        if k[0] != 0:
            continue
        a[(k[2] * ns + k[1]) * per + (k[3] if proto == SET else 0)] = v
    b = np.zeros(R * ns * per, dtype=np.int64)
    for k, v in expected_final_credits(spec).items():
        if k[0] != 0:
            continue
        b[(k[2] * ns + k[1]) * per + (k[3] if proto == SET else 0)] = v * csplit
    return np.concatenate([a, b])
