"""GPU parity of the Reverse All2All combine against the CPU oracle.

Every case compares the HIP path (called through the C ABI) with the oracle
byte for byte, and the final signal arrays with the protocol model's closed
forms.  Sizes: small ragged cases that span several tiles with ragged tails,
edge cases (W=1, one-byte elements, tiles larger than the problem, ring depth
1), and the four combine workloads at their full sizes, in the direct mode
(the default), the staged mode and the two-phase variant.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import moe_all2all_combine_amd as ra2a  # noqa: E402
import oracle  # noqa: E402
import synthgen  # noqa: E402
import expected  # noqa: E402
from combine_harness import CombineCase, opts_for, say  # noqa: E402

pytestmark = pytest.mark.gpu


def expected_signal_array(wl, opts, csplit):
    return expected.expected_signal_array(wl.W, wl.S, wl.H, wl.D, opts, csplit, wl.dtype)


TAKEN = 1 << 63
QUEUED = (ra2a.MODE_STAGED, ra2a.MODE_BULK, ra2a.MODE_PULL)  # modes with work queues


def check_queue_words(q, opts):
    """Staged mode, per group: the home claim counter moved, or (XCD-local sync
    only) another XCD, named in bits 32..39, took the group over and its counter
    moved; every group is marked fully claimed.  Direct mode: untouched."""
    q = q.astype(np.uint64)
    assert len(q) == ra2a.QUEUE_SLOTS == 18
    if opts.mode not in QUEUED:
        # the direct modes touch only the last word: the claim counter of a dynamic
        # schedule, which ends at the number of work items (or stays 0: static)
        assert not q[:17].any(), q
        work = ra2a.rev_all2all_plan(*opts._shape, opts).work_items if hasattr(opts, "_shape") else None
        assert int(q[17]) == 0 or work is None or int(q[17]) == work, (int(q[17]), work)
        return
    assert int(q[16]) == 0xFF and int(q[17]) == 0, q[16:]
    for g, (head, taker) in enumerate(q[:16].reshape(8, 2)):
        head, taker = int(head), int(taker)
        if head & TAKEN:
            assert not opts.agent_sync and opts.mode in QUEUED, \
                f"group {g} taken over, but only the staged XCD-local mode binds groups to XCDs"
            assert 1 <= (head >> 32) & 0xFF <= 8 and taker >= 1, (g, hex(head), taker)
        else:
            assert head >= 1 and taker == 0, (g, head, taker)


def run_and_check(wl, opts, variant="pipelined", inputs=None, want=None, check_signals=True,
                  csplit=None):
    opts._shape = (wl.W, wl.S, wl.H, wl.D, wl.dtype)
    say(f"[case] {variant} {wl.name} W={wl.W} S={wl.S} H={wl.H} D={wl.D} {wl.dtype} "
        f"tile=({opts.tile_s},{opts.tile_h},{opts.tile_d}) proto={opts.protocol} ring={opts.ring}")
    case = CombineCase(wl, opts, two_phase=(variant == "two_phase"))
    try:
        ins = inputs if inputs is not None else synthgen.make_inputs(wl)
        want = want if want is not None else oracle.combine(ins)
        case.upload(ins)
        case.fill_out(0xA5)
        if variant == "two_phase":
            case.run_two_phase()
        else:
            case.run_pipelined()
        torch.cuda.synchronize()
        case.check_device()
        for j in range(wl.W):
            got = case.download(j)
            assert got.tobytes() == want[j].tobytes(), f"rank {j} differs from the oracle"
        if variant == "pipelined" and check_signals:
            cs = csplit if csplit is not None else opts.consumer_split
            exp = expected_signal_array(wl, opts, cs)
            for j in range(wl.W):
                np.testing.assert_array_equal(case.signals(j), exp, err_msg=f"signals of rank {j}")
            check_queue_words(case.queue_words(), opts)
    finally:
        case.close()


SMALL = [
    # (W, S, H, D, dtype, tile, protocol, ring)
    (2, 8, 4, 16, "i32", (8, 4, 16), synthgen.PROTOCOL_SET, 2),
    (3, 37, 2, 40, "bf16", (16, 1, 16), synthgen.PROTOCOL_ADD, 2),
    (3, 37, 2, 40, "bf16", (16, 1, 16), synthgen.PROTOCOL_SET, 1),
    (4, 7, 3, 12, "bf16", (3, 2, 12), synthgen.PROTOCOL_ADD, 1),
    (5, 33, 1, 24, "u8", (8, 1, 7), synthgen.PROTOCOL_ADD, 3),
    (2, 65, 3, 5, "u8", (64, 3, 5), synthgen.PROTOCOL_SET, 2),
    (1, 50, 2, 64, "f32", (16, 2, 64), synthgen.PROTOCOL_ADD, 2),
    (8, 64, 4, 128, "bf16", (16, 1, 128), synthgen.PROTOCOL_ADD, 2),
    (6, 20, 2, 8, "f64", (32, 4, 64), synthgen.PROTOCOL_ADD, 2),   # tiles larger than the problem
    (4, 96, 2, 256, "bf16", (32, 2, 256), synthgen.PROTOCOL_ADD, 8),  # ring deeper than S-blocks
    (16, 9, 3, 32, "f32", (4, 1, 32), synthgen.PROTOCOL_SET, 2),
]


@pytest.mark.parametrize("W,S,H,D,dtype,tile,proto,ring", SMALL)
@pytest.mark.parametrize("csplit", [1, 3])
def test_small_staged(W, S, H, D, dtype, tile, proto, ring, csplit):
    wl = synthgen.small_workload(W, S, H, D, dtype, seed=W * 100 + S, tile=tile, protocol=proto)
    opts = opts_for(wl, ring=ring, consumer_split=csplit, mode=ra2a.MODE_STAGED)
    run_and_check(wl, opts)


@pytest.mark.parametrize("W,S,H,D,dtype,tile,proto,ring", SMALL)
@pytest.mark.parametrize("knobs", [dict(), dict(piece_rows=1), dict(piece_rows=3),
                                   dict(piece_rows=5, wg_per_cu=1),
                                   dict(mode=ra2a.MODE_ROWS), dict(mode=ra2a.MODE_ROWS, unit_rows=1),
                                   dict(mode=ra2a.MODE_ROWS, unit_rows=3)])
def test_small_direct(W, S, H, D, dtype, tile, proto, ring, knobs):
    """The direct modes: per-source pieces (the default; whole tiles, or tiles cut
    into pieces of a few tokens with arrival counters) and row units."""
    wl = synthgen.small_workload(W, S, H, D, dtype, seed=W * 100 + S + 2, tile=tile, protocol=proto)
    opts = opts_for(wl, **knobs)
    run_and_check(wl, opts, csplit=1)


# Row units whose per-source run (H*D*e bytes) relates to the 4 KiB round of
# 256 lanes x 16 bytes in each way the row copy handles: whole rounds per run
# (8 KiB: two; 4 KiB: one), several runs per round (2 KiB, 512 B, with a last,
# partial round when the unit's tokens do not fill it) and neither (6 KiB, 96 B:
# the general plan walk).
ROW_RUNS = [
    (3, 21, 4, 1024, "bf16", (8, 1, 1024), synthgen.PROTOCOL_ADD),
    (4, 19, 2, 1024, "bf16", (8, 2, 1024), synthgen.PROTOCOL_SET),
    (8, 24, 8, 128, "bf16", (8, 1, 128), synthgen.PROTOCOL_ADD),
    (5, 23, 4, 128, "f32", (16, 1, 64), synthgen.PROTOCOL_ADD),
    (4, 30, 2, 128, "bf16", (8, 1, 128), synthgen.PROTOCOL_SET),
    (3, 17, 3, 512, "f32", (8, 1, 512), synthgen.PROTOCOL_ADD),
    (4, 13, 3, 16, "bf16", (4, 1, 16), synthgen.PROTOCOL_ADD),
]


@pytest.mark.parametrize("W,S,H,D,dtype,tile,proto", ROW_RUNS)
@pytest.mark.parametrize("unit_rows", [0, 1, 3, 5])
def test_row_units_run_shapes(W, S, H, D, dtype, tile, proto, unit_rows):
    wl = synthgen.small_workload(W, S, H, D, dtype, seed=W * 31 + S + unit_rows, tile=tile,
                                 protocol=proto)
    opts = opts_for(wl, mode=ra2a.MODE_ROWS, unit_rows=unit_rows)
    run_and_check(wl, opts, csplit=1)


@pytest.mark.parametrize("W,S,H,D,dtype,tile,proto,ring", SMALL[:6])
def test_small_staged_agent_sync(W, S, H, D, dtype, tile, proto, ring):
    wl = synthgen.small_workload(W, S, H, D, dtype, seed=W * 100 + S + 1, tile=tile, protocol=proto)
    opts = opts_for(wl, ring=ring, consumer_split=2, lookahead=2, agent_sync=1,
                    mode=ra2a.MODE_STAGED)
    run_and_check(wl, opts)


@pytest.mark.parametrize("W,S,H,D,dtype,tile,proto,ring", SMALL)
@pytest.mark.parametrize("knobs", [dict(consumer_split=1), dict(consumer_split=2, lookahead=2),
                                   dict(consumer_split=1, agent_sync=1)])
@pytest.mark.parametrize("mode", [ra2a.MODE_BULK, ra2a.MODE_PULL])
def test_small_bulk(W, S, H, D, dtype, tile, proto, ring, knobs, mode):
    """Two-phase layout with per-(S-block, sender) signals; staged at the receiver
    (bulk) or at the sender and pulled by the receiver (pull)."""
    wl = synthgen.small_workload(W, S, H, D, dtype, seed=W * 100 + S + 5, tile=tile, protocol=proto)
    opts = opts_for(wl, mode=mode, **knobs)
    run_and_check(wl, opts, csplit=knobs["consumer_split"])


@pytest.mark.parametrize("W,S,H,D,dtype,tile,proto,ring", SMALL)
def test_small_two_phase(W, S, H, D, dtype, tile, proto, ring):
    wl = synthgen.small_workload(W, S, H, D, dtype, seed=W * 100 + S, tile=tile, protocol=proto)
    run_and_check(wl, opts_for(wl), variant="two_phase")


@pytest.mark.parametrize("mode", [0, ra2a.MODE_ROWS, ra2a.MODE_STAGED])
def test_iota_w2_worked_case(mode):
    wl = synthgen.WORKLOADS["iota_w2_s8_h4_d16_i32"]
    opts = opts_for(wl, consumer_split=1, mode=mode)
    run_and_check(wl, opts)


STAGED = ra2a.MODE_STAGED


@pytest.mark.parametrize("knobs", [
    dict(wg_per_cu=1, mode=STAGED), dict(wg_per_cu=4, mode=STAGED), dict(wg_per_cu=1),
    dict(lookahead=1, mode=STAGED), dict(lookahead=-1, consumer_split=8, mode=STAGED),
    dict(lookahead=1000, ring=3, mode=STAGED),
    dict(agent_sync=1, mode=STAGED), dict(agent_sync=1, lookahead=1, consumer_split=3, mode=STAGED),
    dict(stream_batch=1, mode=STAGED), dict(stream_batch=3, ring=1, mode=STAGED),
    dict(stream_batch=1000, ring=4, mode=STAGED),
    dict(head_merge=1, mode=STAGED), dict(head_merge=2, ring=1, mode=STAGED), dict(head_merge=3),
])
def test_launch_shapes_do_not_change_results(knobs):
    wl = synthgen.small_workload(8, 200, 3, 96, "bf16", seed=5, tile=(32, 1, 96),
                                 protocol=synthgen.PROTOCOL_ADD)
    opts = opts_for(wl, **knobs)
    cs = knobs.get("consumer_split", 1)
    if "consumer_split" not in knobs:
        opts.consumer_split = 1
    run_and_check(wl, opts, csplit=cs)


def test_back_to_back_launches_reset_signals():
    """A second launch on new data must not be satisfied by the first one's signals."""
    wl = synthgen.small_workload(4, 64, 2, 64, "bf16", seed=1, tile=(16, 1, 64),
                                 protocol=synthgen.PROTOCOL_ADD)
    opts = opts_for(wl, consumer_split=2, ring=1, mode=ra2a.MODE_STAGED)
    case = CombineCase(wl, opts)
    try:
        for seed in (1, 2, 3):
            say(f"[case] back-to-back seed={seed}")
            wl2 = synthgen.small_workload(4, 64, 2, 64, "bf16", seed=seed, tile=(16, 1, 64))
            ins = synthgen.make_inputs(wl2)
            case.upload(ins)
            case.run_pipelined()
            torch.cuda.synchronize()
            case.check_device()
            want = oracle.combine(ins)
            for j in range(wl.W):
                assert case.download(j).tobytes() == want[j].tobytes()
            exp = expected_signal_array(wl, opts, 2)
            for j in range(wl.W):
                np.testing.assert_array_equal(case.signals(j), exp)
    finally:
        case.close()


DIRTY = 0x5A  # byte pattern left in the signal array before a launch


@pytest.mark.parametrize("mode", [0, ra2a.MODE_ROWS])
@pytest.mark.parametrize("reset", ["in_launch", "separate", "full_grid"])
def test_direct_reset_clears_dirty_signals(reset, mode):
    """The direct modes zero the signals inside the combine launch (with
    separate_reset, in a launch of its own), also when the persistent grid fills
    every slot the occupancy allows: whatever the signal array held, the data
    signals and counters end at their closed forms and the queue words at 0,
    launch after launch; each in-launch reset leaves its own tag in the reset
    flags."""
    wl = synthgen.small_workload(8, 96, 4, 64, "bf16", seed=11, tile=(16, 1, 64),
                                 protocol=synthgen.PROTOCOL_ADD)
    knobs = {"in_launch": {}, "separate": dict(separate_reset=1), "full_grid": dict(wg_per_cu=64)}
    opts = opts_for(wl, mode=mode, **knobs[reset])
    case = CombineCase(wl, opts)
    dirty = int.from_bytes(bytes([DIRTY]) * 8, "little")
    try:
        tags = []
        for seed in (11, 12, 13):
            say(f"[case] direct reset={reset} seed={seed}")
            case.fill_signals(DIRTY)
            ins = synthgen.make_inputs(synthgen.small_workload(8, 96, 4, 64, "bf16", seed=seed,
                                                               tile=(16, 1, 64)))
            case.upload(ins)
            case.run_pipelined()
            torch.cuda.synchronize()
            case.check_device()
            want = oracle.combine(ins)
            for j in range(wl.W):
                assert case.download(j).tobytes() == want[j].tobytes()
            exp = expected_signal_array(wl, opts, 1)
            for j in range(wl.W):
                np.testing.assert_array_equal(case.signals(j), exp, err_msg=f"signals of rank {j}")
            assert not case.queue_words().any()
            f = [int(x) & (2**64 - 1) for x in case.reset_flags()]
            if reset != "separate":
                nz = next((k for k in range(1, len(f)) if f[k] != f[0]), len(f))
                assert f[0] not in (0, dirty), hex(f[0])
                assert all(x == dirty for x in f[nz:]), "flags past the zeroing workgroups moved"
                tags.append(f[0])
            else:
                assert all(x == dirty for x in f), "a separate reset launch leaves the flags alone"
        if reset != "separate":
            assert len(set(tags)) == len(tags), "every launch has a tag of its own"
    finally:
        case.close()


@pytest.mark.parametrize("mode", [0, ra2a.MODE_ROWS, ra2a.MODE_STAGED])
def test_graph_capture_and_replay(mode):
    """A combine captured in a HIP graph and replayed three times, with eager work
    between the replays (outputs poisoned, signal arrays and control words filled
    with garbage): every replay's output equals the oracle's and its signals the
    eager call's.  Under capture the reset is a launch of its own."""
    W, S, H, D = 4, 96, 4, 64
    wl = synthgen.small_workload(W, S, H, D, "bf16", seed=31, tile=(32, 1, 64))
    case = CombineCase(wl, opts_for(wl, mode=mode, consumer_split=2))
    say(f"[case] graph capture and replay, mode={mode}")
    try:
        ins = synthgen.make_inputs(wl)
        want = oracle.combine(ins)
        case.upload(ins)
        case.run_pipelined()  # the first call on the heap, outside capture
        torch.cuda.synchronize()
        case.check_device()
        eager_sig = [case.signals(j) for j in range(W)]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            case.run_pipelined()
        for rep in range(3):
            case.fill_out(0xA5)
            case.fill_signals(0x5A)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            case.check_device()
            for j in range(W):
                assert case.download(j).tobytes() == want[j].tobytes(), f"replay {rep}, rank {j}"
                np.testing.assert_array_equal(case.signals(j), eager_sig[j], err_msg=f"replay {rep}")
        del g
    finally:
        case.close()


@pytest.mark.parametrize("mode", [ra2a.MODE_DIRECT, ra2a.MODE_STAGED, ra2a.MODE_BULK, ra2a.MODE_PULL])
def test_straggler_timestamps(mode):
    """Per-tile completion clocks under a delayed source: every tile is stamped
    (garbage left in the stamp array is cleared by the combine), and under SET
    (one signal per source and tile) the delayed source's tiles complete later
    on average than the others'."""
    W, S, H, D = 4, 128, 4, 64
    wl = synthgen.small_workload(W, S, H, D, "f32", seed=21, tile=(16, 1, 64),
                                 protocol=synthgen.PROTOCOL_SET)
    lag = 1
    opts = opts_for(wl, mode=mode, straggler_rank=lag, straggler_delay=400, straggler_seed=7,
                    consumer_split=1)
    nt = ra2a.rev_all2all_signal_slots(W, S, H, D, "f32", opts)[0]
    stamps = torch.full((W * nt,), -1, dtype=torch.int64, device="cuda")
    opts.timestamps = stamps.data_ptr()
    say(f"[case] straggler timestamps mode={mode}")
    run_and_check(wl, opts, csplit=1)
    t = stamps.cpu().numpy().view(np.uint64).reshape(W, nt // W, W)  # [dest, tile, source]
    assert (t > 0).all() and (t != np.uint64(2**64 - 1)).all(), "a tile was not stamped"
    t = (t - t.min()).astype(np.float64)
    others = [r for r in range(W) if r != lag]
    assert t[:, :, lag].mean() > t[:, :, others].mean(), (t[:, :, lag].mean(), t[:, :, others].mean())


@pytest.mark.parametrize("proto", [synthgen.PROTOCOL_ADD, synthgen.PROTOCOL_SET])
@pytest.mark.parametrize("unit_rows", [4, 3])
def test_row_units_stamp_every_tile(proto, unit_rows):
    """Row units with completion stamps: every signal tile is stamped, under ADD
    with units adding their shares (4 units per S-block, W = 4) or counting to the
    block's completion (3 units: 16 = 3 + 3 + 3 + 3 + 3 + 1 rows, 6 units), and
    under SET; garbage left in the stamp array is cleared."""
    W, S, H, D = 4, 128, 4, 64
    wl = synthgen.small_workload(W, S, H, D, "f32", seed=23 + unit_rows, tile=(16, 1, 64),
                                 protocol=proto)
    opts = opts_for(wl, mode=ra2a.MODE_ROWS, unit_rows=unit_rows)
    nt = ra2a.rev_all2all_signal_slots(W, S, H, D, "f32", opts)[0]
    stamps = torch.full((W * nt,), -1, dtype=torch.int64, device="cuda")
    opts.timestamps = stamps.data_ptr()
    say(f"[case] row-unit stamps proto={proto} unit_rows={unit_rows}")
    run_and_check(wl, opts, csplit=1)
    t = stamps.cpu().numpy().view(np.uint64)
    assert (t > 0).all() and (t != np.uint64(2**64 - 1)).all(), "a tile was not stamped"


@pytest.mark.parametrize("mode", [0, ra2a.MODE_ROWS, ra2a.MODE_STAGED])
def test_pipelined_equals_two_phase_bitwise(mode):
    """The barrier-synchronised variant as a differential for the signal-pipelined one."""
    wl = synthgen.small_workload(8, 300, 4, 72, "f16", seed=9, tile=(24, 1, 72))
    case = CombineCase(wl, opts_for(wl, consumer_split=2, mode=mode))
    try:
        ins = synthgen.make_inputs(wl)
        case.upload(ins)
        case.run_pipelined()
        torch.cuda.synchronize()
        case.check_device()
        a = [case.download(j) for j in range(wl.W)]
        case.fill_out(0)
        case.run_two_phase()
        torch.cuda.synchronize()
        b = [case.download(j) for j in range(wl.W)]
        for j in range(wl.W):
            assert a[j].tobytes() == b[j].tobytes()
    finally:
        case.close()


def test_special_float_payloads_survive():
    """NaN payloads, -0.0, infinities and subnormals are moved as bytes."""
    W, S, H, D = 4, 16, 2, 64
    wl = synthgen.small_workload(W, S, H, D, "f32", seed=0, tile=(8, 1, 64))
    specials = np.array([0x7FC00001, 0xFFC12345, 0x80000000, 0x7F800000, 0xFF800000, 0x00000001,
                         0x807FFFFF, 0x7FA00000], dtype=np.uint32)
    rng = np.random.default_rng(0)
    ins = [specials[rng.integers(0, len(specials), size=(S * W, H, D))].view(np.float32)
           for _ in range(W)]
    run_and_check(wl, opts_for(wl), inputs=ins)
    run_and_check(wl, opts_for(wl, consumer_split=1, mode=ra2a.MODE_STAGED), inputs=ins)
    run_and_check(wl, opts_for(wl), variant="two_phase", inputs=ins)


# ---- full-size workloads ------------------------------------------------------------

_FULL_CACHE = {}


def full_case(name, variant, **kw):
    wl = synthgen.WORKLOADS[name]
    if name not in _FULL_CACHE:
        _FULL_CACHE.clear()
        say(f"[full] generating {name}")
        ins = synthgen.make_inputs(wl)
        say(f"[full] oracle {name}")
        _FULL_CACHE[name] = (ins, oracle.combine(ins))
    ins, want = _FULL_CACHE[name]
    if variant in ("staged", "bulk", "pull"):
        kw["mode"] = {"staged": ra2a.MODE_STAGED, "bulk": ra2a.MODE_BULK, "pull": ra2a.MODE_PULL}[variant]
        variant = "pipelined"
    elif variant == "rows":
        kw["mode"] = ra2a.MODE_ROWS
        variant = "pipelined"
    elif variant == "whole_tiles":  # one piece per tile and source
        kw["piece_rows"] = wl.tile_s
        variant = "pipelined"
    else:
        kw.pop("consumer_split", None)
    opts = opts_for(wl, consumer_split=kw.pop("consumer_split", 1), **kw)
    run_and_check(wl, opts, variant=variant, inputs=ins, want=want,
                  csplit=None if opts.mode in QUEUED else 1)


@pytest.mark.parametrize("variant", ["pipelined", "rows", "staged", "bulk", "pull", "two_phase"])
def test_full_ep_combine_w8_bf16(variant):
    full_case("ep_combine_w8_s512_h16_d128_bf16", variant)


@pytest.mark.parametrize("variant", ["pipelined", "whole_tiles", "rows", "staged", "bulk", "pull",
                                     "two_phase"])
def test_full_moe_combine_w8_d7168(variant):
    full_case("moe_combine_w8_s4096_h1_d7168_bf16", variant, consumer_split=4)


def test_full_straggler_timestamps():
    """The straggler workload at full size in the default mode, with per-tile
    stamps: every (tile, source) slot is stamped, and the delayed source's tiles
    complete later than the others' at the median."""
    wl = synthgen.WORKLOADS["straggler_w16_s2048_h32_d128_f32"]
    W, S, H, D = wl.W, wl.S, wl.H, wl.D
    lag = synthgen.straggler_rank(wl)
    opts = opts_for(wl, straggler_rank=lag, straggler_delay=1000, straggler_seed=2)
    nt = ra2a.rev_all2all_signal_slots(W, S, H, D, wl.dtype, opts)[0]
    stamps = torch.full((W * nt,), -1, dtype=torch.int64, device="cuda")
    opts.timestamps = stamps.data_ptr()
    if "straggler_w16_s2048_h32_d128_f32" not in _FULL_CACHE:
        _FULL_CACHE.clear()
        say("[full] generating straggler_w16_s2048_h32_d128_f32")
        ins = synthgen.make_inputs(wl)
        _FULL_CACHE["straggler_w16_s2048_h32_d128_f32"] = (ins, oracle.combine(ins))
    ins, want = _FULL_CACHE["straggler_w16_s2048_h32_d128_f32"]
    run_and_check(wl, opts, inputs=ins, want=want, csplit=1)
    t = stamps.cpu().numpy().view(np.uint64).reshape(W, nt // W, W)
    assert (t > 0).all() and (t != np.uint64(2**64 - 1)).all(), "a tile was not stamped"
    t = (t - t.min()).astype(np.float64)
    others = np.delete(t, lag, axis=2)
    assert np.median(t[:, :, lag]) > np.median(others), (np.median(t[:, :, lag]), np.median(others))


@pytest.mark.parametrize("variant", ["pipelined", "staged", "bulk", "pull", "two_phase"])
def test_full_straggler_w16_f32(variant):
    wl = synthgen.WORKLOADS["straggler_w16_s2048_h32_d128_f32"]
    full_case("straggler_w16_s2048_h32_d128_f32", variant,
              straggler_rank=synthgen.straggler_rank(wl), straggler_delay=200, straggler_seed=2)


@pytest.mark.parametrize("variant", ["pipelined", "rows"])
def test_full_straggler_w16_f32_undelayed(variant):
    """The C4 shape without the delay (SET per (tile, source)): the default direct
    mode (dynamically claimed pieces, arrival counters) and row units."""
    full_case("straggler_w16_s2048_h32_d128_f32", variant)
