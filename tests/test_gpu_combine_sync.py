"""GPU tests of what a combine's tile signal guarantees while the launch runs,
of the in-launch reset next to other work, and of the plain entry point.

* A consumer on a second stream waits (ra2a_wait_signal, EQ its final value)
  for one tile of a running combine, copies the tile out, and must find the
  oracle's bytes -- before the combine has finished (checked with events).
* The combine runs while ordinary kernels (large matrix products) occupy the
  device on another stream; its in-launch reset must still complete.
* ra2a_rev_all2all with no options (the plain signature) at the W=2 iota
  worked case and the full W=8 bf16 workload, byte for byte.
Every call goes through the C ABI."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import moe_all2all_combine_amd as ra2a  # noqa: E402
import oracle  # noqa: E402
import synthgen  # noqa: E402
import expected  # noqa: E402
from combine_harness import CombineCase, opts_for, say  # noqa: E402

pytestmark = pytest.mark.gpu


def tile_oracle(case, j, s0, bs):
    """Oracle bytes of out_j rows [s0, s0 + bs): the combine of the sub-problem
    whose destination 0 receives in_r rows j*S + s0 .. of every source."""
    wl = case.wl
    W, S, H, D = wl.W, wl.S, wl.H, wl.D
    sub = []
    for r in range(W):
        rows = case.in_view(r)[j * S + s0: j * S + s0 + bs].cpu().numpy()
        x = np.zeros((bs * W, H, D), dtype=rows.dtype)
        x[:bs] = rows
        sub.append(x)
    return oracle.combine(sub)[0]


@pytest.mark.parametrize("mode", [0, ra2a.MODE_ROWS])
def test_tile_visible_mid_launch(mode):
    """MoE-combine shape (W=8, S=4096, H=1, D=7168, bf16, 32-token tiles): the
    first tile of destination 0 is waited for and read on another stream while the
    1.4 ms combine still runs."""
    W, S, H, D = 8, 4096, 1, 7168
    wl = synthgen.CombineWorkload(name="moe_shape_mid_launch", W=W, S=S, H=H, D=D, dtype="bf16",
                                  dist="bytes", seed=5, tile_s=32, tile_h=1, tile_d=D,
                                  protocol=synthgen.PROTOCOL_ADD)
    opts = opts_for(wl, mode=mode)
    say(f"[case] mid-launch consumer, mode={mode}")
    case = CombineCase(wl, opts, two_phase=False)
    try:
        g = torch.Generator(device="cuda").manual_seed(5)
        for r in range(W):
            v = case.in_view(r)
            v.copy_(torch.randint(-32768, 32767, v.shape, dtype=torch.int16, device="cuda",
                                  generator=g))
        case.fill_out(0xA5)
        nsig = case.n_tile + case.n_credit + case.n_queue
        s1 = torch.cuda.current_stream()
        s2 = torch.cuda.Stream()
        ra2a.signal_reset(case.heap.handle, case.p_sig, nsig, s1)
        ready = torch.cuda.Event()
        ready.record(s1)
        s2.wait_event(ready)
        t0, t_end, t_copy = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        t0.record(s1)
        tile_sig = case.heap.ptr(case.off_sig, 0)  # tile (b=0, head block 0) of destination 0
        ra2a.wait_signal(case.heap.handle, tile_sig, W, ra2a.CMP_EQ, s2)
        with torch.cuda.stream(s2):
            got = case.out_view(0)[0:32].clone()
        t_copy.record(s2)
        case.run_pipelined(s1)
        t_end.record(s1)
        torch.cuda.synchronize()
        case.check_device()
        t_copy_ms, t_end_ms = t0.elapsed_time(t_copy), t0.elapsed_time(t_end)
        say(f"[case] tile copied at {t_copy_ms:.3f} ms, combine ended at {t_end_ms:.3f} ms")
        want = tile_oracle(case, 0, 0, 32)
        assert got.cpu().numpy().tobytes() == want.tobytes(), "the tile read after its signal differs"
        assert t_copy_ms < t_end_ms, "the consumer did not run while the combine was running"
        # and the whole output still matches
        assert int(case.signals(0)[0]) == W
    finally:
        case.close()


@pytest.mark.parametrize("knobs", [dict(), dict(mode=ra2a.MODE_ROWS), dict(wg_per_cu=64),
                                   dict(piece_rows=8)])
def test_in_launch_reset_beside_busy_device(knobs):
    """Large matrix products on another stream occupy the compute units while the
    combine (with its in-launch reset, signals dirty beforehand) is launched: it
    completes with every wait satisfied and the oracle's bytes."""
    wl = synthgen.WORKLOADS["ep_combine_w8_s512_h16_d128_bf16"]
    opts = opts_for(wl, **knobs)
    say(f"[case] in-launch reset beside a busy device {knobs}")
    case = CombineCase(wl, opts, two_phase=False)
    try:
        ins = synthgen.make_inputs(wl)
        case.upload(ins)
        want = oracle.combine(ins)
        a = torch.randn(8192, 8192, device="cuda", dtype=torch.bfloat16)
        b = torch.randn(8192, 8192, device="cuda", dtype=torch.bfloat16)
        s2 = torch.cuda.Stream()
        for rep in range(2):
            case.fill_signals(0x5A)
            case.fill_out(0xA5)
            torch.cuda.synchronize()
            with torch.cuda.stream(s2):
                for _ in range(4):
                    c = torch.matmul(a, b)
            case.run_pipelined()
            torch.cuda.synchronize()
            case.check_device()
            for j in range(wl.W):
                assert case.download(j).tobytes() == want[j].tobytes(), f"rep {rep}, rank {j}"
            exp = expected.expected_signal_array(wl.W, wl.S, wl.H, wl.D, opts, 1, wl.dtype)
            for j in range(wl.W):
                np.testing.assert_array_equal(case.signals(j), exp, err_msg=f"signals of rank {j}")
        del c
    finally:
        case.close()


@pytest.mark.parametrize("name", ["iota_w2_s8_h4_d16_i32", "ep_combine_w8_s512_h16_d128_bf16"])
def test_plain_entry_point_null_options(name):
    """ra2a_rev_all2all (no options): the library's defaults, byte for byte."""
    wl = synthgen.WORKLOADS[name]
    opts = ra2a.Opts()  # what NULL options mean
    say(f"[case] plain rev_all2all {name}")
    case = CombineCase(wl, opts, two_phase=False)
    try:
        ins = synthgen.make_inputs(wl)
        case.upload(ins)
        want = oracle.combine(ins)
        for rep in range(2):
            case.fill_out(0xA5)
            case.fill_signals(0x5A)
            ra2a.rev_all2all(case.p_in, case.p_out, case.p_sig, wl.W, wl.S, wl.H, wl.D, wl.dtype,
                             torch.cuda.current_stream())
            torch.cuda.synchronize()
            case.check_device()
            for j in range(wl.W):
                assert case.download(j).tobytes() == want[j].tobytes(), f"rank {j}"
            exp = expected.expected_signal_array(wl.W, wl.S, wl.H, wl.D, opts, 1, wl.dtype)
            for j in range(wl.W):
                np.testing.assert_array_equal(case.signals(j), exp)
    finally:
        case.close()
