"""GPU parity of the forward All2All (dispatch, the combine's inverse map),
called through the C ABI, against the CPU oracle: out_r[j*S+s, h, d] =
in_j[s, r*H+h, d] byte for byte, every (tile, source) signal at 1, and round
trips through the combine (combine after dispatch returns the input; this
holds at any size, so the MoE-combine-shaped workload is checked that way)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import moe_all2all_combine_amd as ra2a  # noqa: E402
import oracle  # noqa: E402
import synthgen  # noqa: E402
from combine_harness import CombineCase, opts_for, say  # noqa: E402
from expected import expected_signal_array  # noqa: E402

pytestmark = pytest.mark.gpu


def run_dispatch(wl, opts, fill_signals=None):
    W, S, H, D = wl.W, wl.S, wl.H, wl.D
    say(f"[case] dispatch {wl.name} W={W} S={S} H={H} D={D} {wl.dtype} "
        f"tile=({opts.tile_s},{opts.tile_h},{opts.tile_d})")
    case = CombineCase(wl, opts, two_phase=False)
    try:
        ins = [x.reshape(S, H * W, D) for x in synthgen.make_inputs(wl)]  # in_j: (S, H*W, D)
        case.upload([x.reshape(S * W, H, D) for x in ins])
        case.fill_out(0xA5)
        if fill_signals is not None:
            case.fill_signals(fill_signals)
        ra2a.all2all_dispatch_ex(case.p_in, case.p_out, case.p_sig, W, S, H, D, wl.dtype, opts,
                                 torch.cuda.current_stream())
        torch.cuda.synchronize()
        case.check_device()
        want = oracle.dispatch(ins)
        for r in range(W):
            assert case.download(r).tobytes() == want[r].tobytes(), f"rank {r} differs"
        exp = expected_signal_array(W, S, H, D, opts, 1, wl.dtype)
        for r in range(W):
            np.testing.assert_array_equal(case.signals(r), exp, err_msg=f"signals of rank {r}")
    finally:
        case.close()


SMALL = [
    # (W, S, H, D, dtype, tile)
    (2, 8, 4, 16, "i32", (8, 4, 16)),
    (3, 37, 2, 40, "bf16", (16, 1, 16)),
    (4, 7, 3, 12, "bf16", (3, 2, 12)),
    (5, 33, 1, 24, "u8", (8, 1, 7)),
    (1, 50, 2, 64, "f32", (16, 2, 64)),
    (8, 64, 4, 128, "bf16", (16, 1, 128)),
    (6, 20, 2, 8, "f64", (32, 4, 64)),
    (16, 9, 3, 32, "f32", (4, 1, 32)),
]


@pytest.mark.parametrize("W,S,H,D,dtype,tile", SMALL)
@pytest.mark.parametrize("knobs", [{}, dict(agent_sync=1), dict(head_merge=1, separate_reset=1)])
def test_small_dispatch(W, S, H, D, dtype, tile, knobs):
    wl = synthgen.small_workload(W, S, H, D, dtype, seed=W * 100 + S + 9, tile=tile)
    run_dispatch(wl, opts_for(wl, direction=ra2a.DIR_DISPATCH, **knobs))


@pytest.mark.parametrize("W,S,H,D,dtype,tile", SMALL)
@pytest.mark.parametrize("unit_rows", [1, 3, 0])
def test_small_dispatch_row_units(W, S, H, D, dtype, tile, unit_rows):
    """Row units for the dispatch (source j's rows read whole, every destination's
    run written as one contiguous range), on every run shape of SMALL."""
    wl = synthgen.small_workload(W, S, H, D, dtype, seed=W * 100 + S + 19 + unit_rows, tile=tile)
    run_dispatch(wl, opts_for(wl, direction=ra2a.DIR_DISPATCH, mode=ra2a.MODE_ROWS,
                              unit_rows=unit_rows))


@pytest.mark.parametrize("mode", [ra2a.MODE_ROWS, ra2a.MODE_DIRECT])
def test_dispatch_stamps_every_tile(mode):
    """Completion stamps of the dispatch: every (tile, source) slot of every
    destination is stamped, row units (stamped by the unit that completes its
    block, in each destination's row) and pieces alike."""
    W, S, H, D = 4, 96, 4, 64
    wl = synthgen.small_workload(W, S, H, D, "bf16", seed=29, tile=(16, 1, 64))
    opts = opts_for(wl, direction=ra2a.DIR_DISPATCH, mode=mode, unit_rows=5)
    nt = ra2a.rev_all2all_signal_slots(W, S, H, D, "bf16", opts)[0]
    stamps = torch.full((W * nt,), -1, dtype=torch.int64, device="cuda")
    opts.timestamps = stamps.data_ptr()
    run_dispatch(wl, opts)
    t = stamps.cpu().numpy().view(np.uint64)
    assert (t > 0).all() and (t != np.uint64(2**64 - 1)).all(), "a tile was not stamped"


def test_dispatch_clears_dirty_signals():
    wl = synthgen.small_workload(8, 96, 4, 64, "bf16", seed=17, tile=(16, 1, 64))
    run_dispatch(wl, opts_for(wl, direction=ra2a.DIR_DISPATCH), fill_signals=0x5A)


@pytest.mark.parametrize("mode", [0, ra2a.MODE_DIRECT])
def test_full_ep_combine_shape_dispatch(mode):
    wl = synthgen.WORKLOADS["ep_combine_w8_s512_h16_d128_bf16"]
    opts = opts_for(wl, direction=ra2a.DIR_DISPATCH, mode=mode)
    if mode == 0:  # the default on this shape: row units
        assert ra2a.rev_all2all_plan(wl.W, wl.S, wl.H, wl.D, wl.dtype, opts).mode == ra2a.MODE_ROWS
    run_dispatch(wl, opts)


@pytest.mark.parametrize("name", ["ep_combine_w8_s512_h16_d128_bf16",
                                  "moe_combine_w8_s4096_h1_d7168_bf16"])
def test_round_trip_combine_after_dispatch(name):
    """dispatch(x) then combine gives x back bit for bit, at full size, on the GPU."""
    wl = synthgen.WORKLOADS[name]
    W, S, H, D = wl.W, wl.S, wl.H, wl.D
    say(f"[case] round trip {name}")
    opts = opts_for(wl)
    dopts = opts_for(wl, direction=ra2a.DIR_DISPATCH)
    n_sig = max(sum(ra2a.rev_all2all_signal_slots(W, S, H, D, wl.dtype, o)) for o in (opts, dopts))
    nb = wl.bytes_per_rank
    heap = ra2a.SymmHeap(W, 3 * nb + n_sig * 128 + (1 << 20))
    try:
        o_x, o_mid, o_back = heap.alloc(nb), heap.alloc(nb), heap.alloc(nb)
        o_sig = heap.alloc(n_sig * 128)
        g = torch.Generator(device="cuda").manual_seed(3)
        for r in range(W):
            heap.view(o_x, (nb // 4,), torch.int32, r).copy_(
                torch.randint(-2**31, 2**31 - 1, (nb // 4,), generator=g, device="cuda",
                              dtype=torch.int32))
            heap.view(o_back, (nb,), torch.uint8, r).fill_(0xA5)
        st = torch.cuda.current_stream()
        ra2a.all2all_dispatch_ex(heap.ptr(o_x), heap.ptr(o_mid), heap.ptr(o_sig), W, S, H, D,
                                 wl.dtype, dopts, st)
        ra2a.rev_all2all_ex(heap.ptr(o_mid), heap.ptr(o_back), heap.ptr(o_sig), W, S, H, D,
                            wl.dtype, opts, st)
        torch.cuda.synchronize()
        assert ra2a.check(heap.handle) == ra2a.OK, ra2a.last_error()
        for r in range(W):
            assert torch.equal(heap.view(o_x, (nb,), torch.uint8, r),
                               heap.view(o_back, (nb,), torch.uint8, r)), f"rank {r}"
    finally:
        heap.close()
