"""The pipelined kernel's own address arithmetic and work queues, run on the
host (``ra2a_debug_emulate_pipelined``): every access inside its buffer, each
queue holding every piece and consumer item once, every wait already holding
when its task comes up in queue order (the kernel's deadlock-freedom
argument), and the bytes moved equal to the oracle's combine, with the signal
arrays equal to the protocol model's closed forms.  No GPU needed."""
import numpy as np
import pytest

import moe_all2all_combine_amd as ra2a
import oracle
import synthgen
from expected import expected_signal_array

P_ADD = synthgen.PROTOCOL_ADD
P_SET = synthgen.PROTOCOL_SET

CASES = [
    # W, S, H, D, dtype, (tile_s, tile_h, tile_d), protocol, ring, csplit, lookahead
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


def staged_opts(tile, proto, **kw):
    return ra2a.Opts(tile_s=tile[0], tile_h=tile[1], tile_d=tile[2],
                     protocol=ra2a.PROTO_SET if proto == P_SET else ra2a.PROTO_ADD,
                     mode=ra2a.MODE_STAGED, **kw)


def check_emulation(W, S, H, D, dtype, opts, csplit, seed, cus=256, per_cu=2):
    wl = synthgen.small_workload(W, S, H, D, dtype, seed=seed, tile=(opts.tile_s, opts.tile_h,
                                                                     opts.tile_d))
    ins = synthgen.make_inputs(wl)
    outs, sigs = ra2a.debug_emulate_pipelined(ins, W, S, H, D, dtype, opts, cus, per_cu)
    want = oracle.combine(ins)
    exp = expected_signal_array(W, S, H, D, opts, csplit, dtype)
    for j in range(W):
        assert outs[j].tobytes() == want[j].tobytes(), f"rank {j}"
        np.testing.assert_array_equal(sigs[j][:len(exp)].astype(np.int64), exp)
        assert len(sigs[j]) == len(exp) + ra2a.QUEUE_SLOTS + ra2a.RESET_FLAGS
        assert not sigs[j][len(exp):].any()


@pytest.mark.parametrize("W,S,H,D,dtype,tile,proto,ring,csplit,lookahead", CASES)
@pytest.mark.parametrize("cus,per_cu", [(256, 2), (256, 1), (8, 1)])
def test_emulated_kernel_matches_oracle(W, S, H, D, dtype, tile, proto, ring, csplit, lookahead,
                                        cus, per_cu):
    opts = staged_opts(tile, proto, ring=ring, consumer_split=csplit, lookahead=lookahead,
                       wg_per_cu=per_cu)
    check_emulation(W, S, H, D, dtype, opts, csplit, seed=S + W, cus=cus, per_cu=per_cu)


@pytest.mark.parametrize("cus,per_cu", [(1, 1), (2, 1), (3, 2)])
def test_emulated_tiny_devices(cus, per_cu):
    """The queues make any number of resident workgroups enough."""
    opts = staged_opts((8, 1, 8), P_ADD, ring=1, consumer_split=2)
    check_emulation(8, 16, 16, 8, "bf16", opts, 2, seed=4, cus=cus, per_cu=per_cu)


@pytest.mark.parametrize("stream_batch", [1, 2, 3, 1000])
@pytest.mark.parametrize("W,S,H,D,tile,proto,ring", [
    (8, 200, 6, 96, (32, 1, 96), P_ADD, 2),
    (5, 70, 4, 64, (16, 2, 32), P_SET, 3),
    (16, 64, 8, 32, (16, 1, 32), P_ADD, 1),
])
def test_emulated_stream_batches(stream_batch, W, S, H, D, tile, proto, ring):
    opts = staged_opts(tile, proto, ring=ring, consumer_split=2, stream_batch=stream_batch)
    check_emulation(W, S, H, D, "bf16", opts, 2, seed=7)


@pytest.mark.parametrize("lookahead", [-1, 0, 1, 2, 5, 1000])
@pytest.mark.parametrize("W,S,H,D,tile,proto,ring,stream_batch", [
    (8, 200, 6, 96, (32, 1, 96), P_ADD, 2, 2),
    (5, 70, 4, 64, (16, 2, 32), P_SET, 3, 1),
    (16, 64, 8, 32, (16, 1, 32), P_ADD, 1, 3),
])
def test_emulated_lookahead(lookahead, W, S, H, D, tile, proto, ring, stream_batch):
    """Any requested lookahead is capped so that no wait points forward."""
    opts = staged_opts(tile, proto, ring=ring, consumer_split=3, lookahead=lookahead,
                       stream_batch=stream_batch)
    check_emulation(W, S, H, D, "bf16", opts, 3, seed=8)


@pytest.mark.parametrize("W,S,H,D,dtype,tile,proto", [
    (3, 37, 2, 40, "bf16", (16, 1, 16), P_ADD), (3, 37, 2, 40, "bf16", (16, 1, 16), P_SET),
    (8, 512, 16, 128, "bf16", (64, 1, 128), P_ADD), (16, 64, 32, 128, "f32", (64, 1, 128), P_SET),
    (2, 8, 4, 16, "i32", (8, 4, 16), P_SET), (1, 9, 3, 7, "u8", (4, 2, 3), P_ADD),
])
def test_emulated_direct_mode(W, S, H, D, dtype, tile, proto):
    opts = ra2a.Opts(tile_s=tile[0], tile_h=tile[1], tile_d=tile[2],
                     protocol=ra2a.PROTO_SET if proto == P_SET else ra2a.PROTO_ADD)
    assert opts.mode == 0  # the default: direct mode, per-source pieces
    assert ra2a.rev_all2all_workspace_bytes(W, S, H, D, dtype, opts) == 0
    check_emulation(W, S, H, D, dtype, opts, 1, seed=3)
    opts.mode = ra2a.MODE_DIRECT
    check_emulation(W, S, H, D, dtype, opts, 1, seed=3)
    for pr in (1, 3, tile[0] // 2 or 1):  # tiles cut into pieces: arrival counters
        opts.piece_rows = pr
        check_emulation(W, S, H, D, dtype, opts, 1, seed=3)


@pytest.mark.parametrize("unit_rows", [0, 1, 2, 3, 5, 64, 1000])
@pytest.mark.parametrize("W,S,H,D,dtype,tile,proto", [
    (3, 37, 2, 40, "bf16", (16, 1, 16), P_ADD), (3, 37, 2, 40, "bf16", (16, 1, 16), P_SET),
    (8, 512, 16, 128, "bf16", (64, 1, 128), P_ADD), (16, 64, 32, 128, "f32", (64, 1, 128), P_SET),
    (2, 8, 4, 16, "i32", (8, 4, 16), P_SET), (1, 9, 3, 7, "u8", (4, 2, 3), P_ADD),
    (8, 96, 1, 7168, "bf16", (32, 1, 7168), P_ADD), (5, 33, 3, 12, "u8", (7, 2, 5), P_SET),
])
def test_emulated_row_units(unit_rows, W, S, H, D, dtype, tile, proto):
    """Row units: every output row written once by one unit, the bytes equal the
    oracle's, every signal tile ends at W (ADD) or 1 (SET) and every S-block's
    arrival counter at its unit count (the protocol model's closed forms)."""
    opts = ra2a.Opts(tile_s=tile[0], tile_h=tile[1], tile_d=tile[2], unit_rows=unit_rows,
                     mode=ra2a.MODE_ROWS,
                     protocol=ra2a.PROTO_SET if proto == P_SET else ra2a.PROTO_ADD)
    check_emulation(W, S, H, D, dtype, opts, 1, seed=5)


def test_row_units_rejected_for_straggler():
    # row units serve the dispatch too; a delayed straggler source needs pieces
    p = ra2a.rev_all2all_plan(4, 64, 2, 64, "bf16",
                              ra2a.Opts(mode=ra2a.MODE_ROWS, direction=ra2a.DIR_DISPATCH))
    assert p.mode == ra2a.MODE_ROWS
    with pytest.raises(ra2a.Ra2aError) as e:
        ra2a.rev_all2all_signal_slots(4, 64, 2, 64, "bf16",
                                      ra2a.Opts(mode=ra2a.MODE_ROWS, straggler_rank=1,
                                                straggler_delay=10))
    assert e.value.code == ra2a.EINVAL
    with pytest.raises(ra2a.Ra2aError):
        ra2a.rev_all2all_signal_slots(4, 64, 2, 64, "bf16", ra2a.Opts(unit_rows=-1))
    with pytest.raises(ra2a.Ra2aError):
        ra2a.rev_all2all_signal_slots(4, 64, 2, 64, "bf16", ra2a.Opts(piece_rows=-1))
    assert ra2a.rev_all2all_plan(4, 64, 2, 64, "bf16", ra2a.Opts(mode=ra2a.MODE_ROWS)).credit_slots == 1


@pytest.mark.parametrize("head_merge", [1, 2, 3, 16])
@pytest.mark.parametrize("W,S,H,D,dtype,tile,proto,mode", [
    (4, 70, 7, 64, "bf16", (16, 1, 64), P_ADD, ra2a.MODE_STAGED),
    (3, 33, 6, 40, "bf16", (8, 2, 40), P_SET, ra2a.MODE_STAGED),
    (4, 70, 7, 64, "bf16", (16, 1, 64), P_SET, ra2a.MODE_DIRECT),
    (2, 20, 5, 48, "f32", (8, 1, 16), P_ADD, ra2a.MODE_STAGED),
])
def test_emulated_head_merge(head_merge, W, S, H, D, dtype, tile, proto, mode):
    opts = ra2a.Opts(tile_s=tile[0], tile_h=tile[1], tile_d=tile[2],
                     protocol=ra2a.PROTO_SET if proto == P_SET else ra2a.PROTO_ADD, ring=2,
                     consumer_split=2, head_merge=head_merge, mode=mode)
    check_emulation(W, S, H, D, dtype, opts, 2, seed=11)


# ---- the dispatch (the combine's inverse map) ------------------------------------

DISPATCH_CASES = [
    # W, S, H, D, dtype, (tile_s, tile_h, tile_d)
    (2, 8, 4, 16, "i32", (8, 4, 16)),
    (3, 37, 2, 40, "bf16", (16, 1, 16)),
    (4, 7, 3, 12, "bf16", (3, 2, 12)),
    (5, 33, 1, 24, "u8", (8, 1, 7)),
    (1, 50, 2, 64, "f32", (16, 2, 64)),
    (6, 20, 2, 8, "f64", (32, 4, 64)),
    (16, 9, 3, 32, "f32", (4, 1, 32)),
    (8, 512, 16, 128, "bf16", (64, 1, 128)),
    (8, 128, 1, 7168, "bf16", (32, 1, 7168)),
]


@pytest.mark.parametrize("W,S,H,D,dtype,tile", DISPATCH_CASES)
@pytest.mark.parametrize("head_merge", [0, 1, 3])
def test_emulated_dispatch_matches_oracle(W, S, H, D, dtype, tile, head_merge):
    """The kernel's dispatch geometry moves exactly the oracle's bytes, every
    (tile, source) signal ends at 1, and (tiles cut into pieces) every arrival
    counter at its closed form."""
    opts = ra2a.Opts(tile_s=tile[0], tile_h=tile[1], tile_d=tile[2], head_merge=head_merge,
                     direction=ra2a.DIR_DISPATCH)
    wl = synthgen.small_workload(W, S, H, D, dtype, seed=S + 3 * W, tile=tile)
    ins = [x.reshape(S, H * W, D) for x in synthgen.make_inputs(wl)]  # in_j: (S, H*W, D)
    outs, sigs = ra2a.debug_emulate_pipelined(ins, W, S, H, D, dtype, opts)
    want = oracle.dispatch(ins)
    exp = expected_signal_array(W, S, H, D, opts, 1, dtype)
    n_a = W * -(-S // tile[0]) * -(-H // tile[1]) * -(-D // tile[2])
    assert (exp[:n_a] == 1).all()
    assert len(exp) == n_a + ra2a.rev_all2all_signal_slots(W, S, H, D, dtype, opts)[1]
    for r in range(W):
        assert outs[r].tobytes() == want[r].tobytes(), f"rank {r}"
        np.testing.assert_array_equal(sigs[r][:len(exp)].astype(np.int64), exp)
        assert not sigs[r][len(exp):].any()


@pytest.mark.parametrize("W,S,H,D,dtype,tile", DISPATCH_CASES)
@pytest.mark.parametrize("unit_rows", [0, 1, 3, 5])
def test_emulated_dispatch_row_units(W, S, H, D, dtype, tile, unit_rows):
    """Dispatch row units (source j's rows, every destination's run): the
    oracle's bytes, every (tile, source) signal at 1 in every destination's
    slice, every S-block counter at its unit count."""
    opts = ra2a.Opts(tile_s=tile[0], tile_h=tile[1], tile_d=tile[2], unit_rows=unit_rows,
                     mode=ra2a.MODE_ROWS, direction=ra2a.DIR_DISPATCH)
    assert ra2a.rev_all2all_plan(W, S, H, D, dtype, opts).mode == ra2a.MODE_ROWS
    wl = synthgen.small_workload(W, S, H, D, dtype, seed=S + 5 * W + unit_rows, tile=tile)
    ins = [x.reshape(S, H * W, D) for x in synthgen.make_inputs(wl)]
    outs, sigs = ra2a.debug_emulate_pipelined(ins, W, S, H, D, dtype, opts)
    want = oracle.dispatch(ins)
    exp = expected_signal_array(W, S, H, D, opts, 1, dtype)
    n_a = W * -(-S // tile[0]) * -(-H // tile[1]) * -(-D // tile[2])
    assert (exp[:n_a] == 1).all() and len(exp) == n_a + -(-S // tile[0])
    for r in range(W):
        assert outs[r].tobytes() == want[r].tobytes(), f"rank {r}"
        np.testing.assert_array_equal(sigs[r][:len(exp)].astype(np.int64), exp)
        assert not sigs[r][len(exp):].any()


@pytest.mark.parametrize("mode", [ra2a.MODE_STAGED, ra2a.MODE_BULK, ra2a.MODE_PULL])
def test_dispatch_rejects_staged_mode(mode):
    opts = ra2a.Opts(direction=ra2a.DIR_DISPATCH, mode=mode)
    with pytest.raises(ra2a.Ra2aError) as e:
        ra2a.rev_all2all_signal_slots(4, 64, 2, 64, "bf16", opts)
    assert e.value.code == ra2a.EINVAL
    with pytest.raises(ra2a.Ra2aError):
        ra2a.rev_all2all_signal_slots(4, 64, 2, 64, "bf16", ra2a.Opts(mode=6))
    with pytest.raises(ra2a.Ra2aError):
        ra2a.rev_all2all_signal_slots(4, 64, 2, 64, "bf16", ra2a.Opts(direction=2))


# ---- the bulk mode: two-phase layout with fine-grained signals --------------------

@pytest.mark.parametrize("W,S,H,D,dtype,tile,proto,ring,csplit,lookahead", CASES)
@pytest.mark.parametrize("cus,per_cu", [(256, 2), (8, 1)])
@pytest.mark.parametrize("mode", [ra2a.MODE_BULK, ra2a.MODE_PULL])
def test_emulated_bulk_matches_oracle(W, S, H, D, dtype, tile, proto, ring, csplit, lookahead,
                                      cus, per_cu, mode):
    """Every sender's segment lands in the [W][S][H][D] staging (the receiver's,
    or in pull mode the sender's own), each consumer unit waits only for its
    (S-block, sender) signal, and the bytes equal the oracle's; every region-A
    slot ends at 1 and there is no region B."""
    opts = ra2a.Opts(tile_s=tile[0], tile_h=tile[1], tile_d=tile[2], mode=mode,
                     consumer_split=csplit, lookahead=lookahead, wg_per_cu=per_cu)
    nt, nc, _ = ra2a.rev_all2all_signal_slots(W, S, H, D, dtype, opts)
    assert nc == 0 and nt == W * -(-S // tile[0]) * -(-H // tile[1]) * -(-D // tile[2])
    # per slice: one (S, H, D) segment per sender
    assert ra2a.rev_all2all_workspace_bytes(W, S, H, D, dtype, opts) == W * S * H * D * \
        synthgen.small_workload(W, S, H, D, dtype, seed=0, tile=tile).elem_bytes
    check_emulation(W, S, H, D, dtype, opts, csplit, seed=S + W + 1, cus=cus, per_cu=per_cu)


@pytest.mark.parametrize("mode", [ra2a.MODE_BULK, ra2a.MODE_PULL])
def test_bulk_staging_over_4gib_needs_agent_sync(mode):
    big = (16, 16384, 32, 128, "f32")  # 16 senders x 16384 x 32 x 128 x 4 B = 4 GiB per slice
    with pytest.raises(ra2a.Ra2aError) as e:
        ra2a.rev_all2all_signal_slots(*big, ra2a.Opts(mode=mode))
    assert e.value.code == ra2a.EINVAL and "agent_sync" in str(e.value)
    nt, nc, _ = ra2a.rev_all2all_signal_slots(*big, ra2a.Opts(mode=mode, agent_sync=1))
    assert nc == 0
