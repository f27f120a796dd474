"""The pipelined kernel's own address arithmetic and launch partition, run on
the host (``ra2a_debug_emulate_pipelined``): every access inside its buffer,
roles and work lists partitioning the work, every wait satisfiable in
S-block order, and the bytes moved equal to the oracle's combine, with the
signal arrays equal to the protocol model's closed forms.  No GPU needed."""
import numpy as np
import pytest

import moe_all2all_combine_amd as ra2a
import oracle
import synthgen
from expected import expected_signal_array

P_ADD = synthgen.PROTOCOL_ADD
P_SET = synthgen.PROTOCOL_SET

CASES = [
    # W, S, H, D, dtype, (tile_s, tile_h, tile_d), protocol, ring, csplit, pbatch
    (2, 8, 4, 16, "i32", (8, 4, 16), P_SET, 2, 1, 1),
    (3, 37, 2, 40, "bf16", (16, 1, 16), P_ADD, 2, 3, 2),
    (3, 37, 2, 40, "bf16", (16, 1, 16), P_SET, 1, 2, 5),
    (4, 7, 3, 12, "bf16", (3, 2, 12), P_ADD, 1, 1, 16),
    (5, 33, 1, 24, "u8", (8, 1, 7), P_ADD, 3, 4, 3),
    (2, 65, 3, 5, "u8", (64, 3, 5), P_SET, 2, 1, 1),
    (1, 50, 2, 64, "f32", (16, 2, 64), P_ADD, 2, 2, 4),
    (8, 64, 4, 128, "bf16", (16, 1, 128), P_ADD, 2, 1, 4),
    (6, 20, 2, 8, "f64", (32, 4, 64), P_ADD, 2, 1, 1),
    (4, 96, 2, 256, "bf16", (32, 2, 256), P_ADD, 8, 2, 2),
    (16, 9, 3, 32, "f32", (4, 1, 32), P_SET, 2, 3, 7),
    # the workloads' tilings at reduced S
    (8, 512, 16, 128, "bf16", (64, 1, 128), P_ADD, 2, 1, 4),
    (8, 128, 1, 7168, "bf16", (32, 1, 7168), P_ADD, 2, 4, 1),
    (16, 128, 32, 128, "f32", (64, 1, 128), P_SET, 2, 1, 2),
]


@pytest.mark.parametrize("W,S,H,D,dtype,tile,proto,ring,csplit,pbatch", CASES)
@pytest.mark.parametrize("cus,per_cu", [(256, 2), (256, 1), (8, 1)])
def test_emulated_kernel_matches_oracle(W, S, H, D, dtype, tile, proto, ring, csplit, pbatch, cus,
                                        per_cu):
    wl = synthgen.small_workload(W, S, H, D, dtype, seed=S + W, tile=tile, protocol=proto)
    ins = synthgen.make_inputs(wl)
    opts = ra2a.Opts(tile_s=tile[0], tile_h=tile[1], tile_d=tile[2],
                     protocol=ra2a.PROTO_SET if proto == P_SET else ra2a.PROTO_ADD, ring=ring,
                     consumer_split=csplit, producer_batch=pbatch, wg_per_cu=per_cu)
    outs, sigs = ra2a.debug_emulate_pipelined(ins, W, S, H, D, dtype, opts, cus, per_cu)
    want = oracle.combine(ins)
    exp = expected_signal_array(W, S, H, D, opts, csplit)
    for j in range(W):
        assert outs[j].tobytes() == want[j].tobytes(), f"rank {j}"
        np.testing.assert_array_equal(sigs[j].astype(np.int64), exp)


def test_emulator_rejects_device_too_small():
    wl = synthgen.small_workload(8, 16, 16, 8, "bf16", tile=(8, 1, 8))
    ins = synthgen.make_inputs(wl)
    with pytest.raises(ra2a.Ra2aError) as e:
        ra2a.debug_emulate_pipelined(ins, 8, 16, 16, 8, "bf16", None, 2, 1)
    assert e.value.code == ra2a.EUNSUPPORTED


@pytest.mark.parametrize("stream_batch", [1, 2, 3, 1000])
@pytest.mark.parametrize("W,S,H,D,tile,proto,ring", [
    (8, 200, 6, 96, (32, 1, 96), P_ADD, 2),
    (5, 70, 4, 64, (16, 2, 32), P_SET, 3),
    (16, 64, 8, 32, (16, 1, 32), P_ADD, 1),
])
def test_emulated_stream_batches(stream_batch, W, S, H, D, tile, proto, ring):
    wl = synthgen.small_workload(W, S, H, D, "bf16", seed=7, tile=tile, protocol=proto)
    ins = synthgen.make_inputs(wl)
    opts = ra2a.Opts(tile_s=tile[0], tile_h=tile[1], tile_d=tile[2],
                     protocol=ra2a.PROTO_SET if proto == P_SET else ra2a.PROTO_ADD, ring=ring,
                     consumer_split=2, producer_batch=3, stream_batch=stream_batch)
    outs, sigs = ra2a.debug_emulate_pipelined(ins, W, S, H, D, "bf16", opts, 256, 2)
    want = oracle.combine(ins)
    exp = expected_signal_array(W, S, H, D, opts, 2)
    for j in range(W):
        assert outs[j].tobytes() == want[j].tobytes(), f"rank {j}"
        np.testing.assert_array_equal(sigs[j].astype(np.int64), exp)
