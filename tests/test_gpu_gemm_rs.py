"""GPU parity of the GEMM + ReduceScatter (through the C ABI) against the fp64 oracle.

* Integer inputs in {-1, 0, 1}: every fp32 accumulation and every fp32 sum of
  partials is an integer below 2^24, hence exact, and the bf16 rounding of an
  integer partial is the oracle's rounding of the same value; so out_j must equal
  the oracle's sum rounded to bf16 (nearest even) bit for bit: with fp32
  partials (the default) its exact sum, with bf16 partials its sum of rounded
  partials.
* Normal inputs, fp32 partials: max relative error <= 1e-2 against the exact
  fp64 sum, with the floor 0.01 * RMS(ref) (oracle/gemm.py ``rel_error``).
* Normal inputs, bf16 partials: each of the W partials is rounded once (error
  <= 2^-9 |p_r|) and the result once more (<= 2^-9 |out|); fp32 accumulation
  and the fp32 sum add far less than the same again, so elementwise
  |out - ref| <= 2^-8 (sum_r |p_r| + |ref|), p_r the exact partials.
* Every (tile, source) signal ends at 1.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import moe_all2all_combine_amd as ra2a  # noqa: E402
import synthgen  # noqa: E402
from oracle import gemm  # noqa: E402

from combine_harness import say  # noqa: E402

pytestmark = pytest.mark.gpu


def run_gemm_rs(a_bits, bt_bits, flags=0, dirty_signals=False, calls=1, caller_reset=False):
    """Run `calls` back-to-back calls on the same buffers (the signal array keeps
    the previous call's values unless the call resets it); with caller_reset the
    signals are zeroed by ra2a_signal_reset and the calls pass RS_SKIP_RESET."""
    W = len(a_bits)
    m, K = a_bits[0].shape
    N = bt_bits[0].shape[0]
    mj = m // W
    nt, nq, pbytes = ra2a.gemm_rs_sizes(W, m, K, N, flags)
    nsig = nt + nq
    na, nb, no = m * K * 2, N * K * 2, mj * N * 2
    heap = ra2a.SymmHeap(W, na + nb + pbytes + no + nsig * 128 + (1 << 16))
    try:
        oa, ob, op = heap.alloc(na), heap.alloc(nb), heap.alloc(pbytes)
        oo, osg = heap.alloc(no), heap.alloc(nsig * 128)
        for r in range(W):
            heap.view(oa, (m, K), torch.int16, r).copy_(torch.from_numpy(a_bits[r].view(np.int16)))
            heap.view(ob, (N, K), torch.int16, r).copy_(torch.from_numpy(bt_bits[r].view(np.int16)))
            heap.view(op, (pbytes,), torch.uint8, r).fill_(0xFF)   # NaN poison in the partials
            heap.view(oo, (mj, N), torch.int16, r).fill_(0x7FC1)  # NaN poison in the output
            if dirty_signals:
                heap.view(osg, (nsig * 128,), torch.uint8, r).fill_(0x5A)
        torch.cuda.synchronize()
        st = torch.cuda.current_stream()
        for _ in range(calls):
            f = flags
            if caller_reset:
                ra2a.signal_reset(heap.handle, heap.ptr(osg), nsig, st)
                f |= ra2a.RS_SKIP_RESET
            ra2a.gemm_rs(heap.ptr(oa), heap.ptr(ob), heap.ptr(op), heap.ptr(oo), heap.ptr(osg), W, m,
                         K, N, f, st)
        torch.cuda.synchronize()
        rc = ra2a.check(heap.handle)
        assert rc == ra2a.OK, ra2a.last_error()
        outs = [heap.view(oo, (mj, N), torch.int16, j).cpu().numpy().view(np.uint16) for j in range(W)]
        sigs = [heap.view(osg, (nsig, ra2a.SIG_STRIDE_U64), torch.int64, j)[:nt, 0].cpu().numpy()
                for j in range(W)]
        return outs, sigs
    finally:
        heap.close()


EXACT = [
    # W, m, K, N
    (8, 512, 512, 512),
    (3, 300, 72, 200),
    (3, 300, 72, 202),       # N not a multiple of 4: the epilogue's one-column path
    (3, 300, 72, 204),       # N a multiple of 4, not of 8: fp32 vectors, bf16 one column
    (1, 5, 8, 8),            # W = 1: a plain GEMM
    (16, 16 * 130, 64, 264),  # more ranks than XCDs, ragged tiles
    (2, 2 * 520, 1032, 776),
    (5, 5 * 40, 4096, 16),   # long K, narrow N
    (2, 2 * 2048, 64, 2304),  # 72 tiles per destination: several queue blocks, the last ragged
    (3, 3 * 96, 192, 136),   # three 64-k stages: the one refill of the ring
    (2, 2 * 64, 128, 64),    # two whole stages, no refill
]


BF16P = ra2a.RS_BF16_PARTIALS
FLAGS = [0, ra2a.RS_AGENT_SYNC, BF16P, BF16P | ra2a.RS_AGENT_SYNC]


@pytest.mark.parametrize("W,m,K,N", EXACT)
@pytest.mark.parametrize("flags", FLAGS)
def test_integer_inputs_bit_exact(W, m, K, N, flags):
    say(f"[case] gemm_rs integer W={W} m={m} K={K} N={N} flags={flags}")
    a, bt = synthgen.make_gemm_rs_inputs(m=m, K=K, N=N, W=W, integer=True)
    outs, sigs = run_gemm_rs(a, bt, flags)
    ref = gemm.gemm_rs_ref(a, bt, round_partials=bool(flags & BF16P))
    for j in range(W):
        np.testing.assert_array_equal(outs[j], gemm.f64_to_bf16_rne_bits(ref[j]),
                                      err_msg=f"rank {j}")
        assert (sigs[j] == 1).all(), sigs[j]


@pytest.mark.parametrize("caller_reset", [False, True])
def test_back_to_back_calls_and_caller_reset(caller_reset):
    """Three calls in a row on one signal array (each reset by the library, or by
    the caller with RS_SKIP_RESET): the output and the signals are those of one call."""
    W, m, K, N = 4, 4 * 300, 136, 520
    say(f"[case] gemm_rs back-to-back caller_reset={caller_reset}")
    a, bt = synthgen.make_gemm_rs_inputs(m=m, K=K, N=N, W=W, integer=True)
    outs, sigs = run_gemm_rs(a, bt, 0, dirty_signals=True, calls=3, caller_reset=caller_reset)
    ref = gemm.gemm_rs_ref(a, bt)
    for j in range(W):
        np.testing.assert_array_equal(outs[j], gemm.f64_to_bf16_rne_bits(ref[j]), err_msg=f"rank {j}")
        assert (sigs[j] == 1).all(), sigs[j]


def test_integer_partials_that_round():
    """K = 1024 with inputs in {-1, 0, 1}: some partials exceed 256 in magnitude and
    are rounded by the bf16 partial path, exactly as the oracle rounds them."""
    say("[case] gemm_rs integer partials beyond 256, W=2 m=512 K=1024 N=256")
    W, m, K, N = 2, 512, 1024, 256
    # ones in the first 300 columns of half the rows make partials of 300 or so
    a, bt = synthgen.make_gemm_rs_inputs(m=m, K=K, N=N, W=W, integer=True)
    one = np.uint16(0x3F80)
    for r in range(W):
        a[r][::2, :300] = one
        bt[r][:, :300] = one
    outs, _ = run_gemm_rs(a, bt, BF16P)
    ref = gemm.gemm_rs_ref(a, bt, round_partials=True)
    exact = gemm.gemm_rs_ref(a, bt)
    differs = False
    for j in range(W):
        np.testing.assert_array_equal(outs[j], gemm.f64_to_bf16_rne_bits(ref[j]), err_msg=f"rank {j}")
        differs |= not np.array_equal(gemm.f64_to_bf16_rne_bits(exact[j]), outs[j])
    assert differs  # the case does exercise the partials' rounding


def abs_partials_rows(a, bt, j, rows):
    """sum_r |x1_r @ x2_r| on rows `rows` of out_j, from the oracle's per-rank products."""
    mj = a[0].shape[0] // len(a)
    idx = j * mj + np.asarray(rows)
    return sum(np.abs(gemm.gemm_rs_rows_ref([x], [y], 0, idx)) for x, y in zip(a, bt))


def check_outputs(a, bt, outs, flags, j, rows, ref):
    got = gemm.bf16_bits_to_f64(outs[j][rows])
    if flags & BF16P:
        bound = 2.0 ** -8 * (abs_partials_rows(a, bt, j, rows) + np.abs(ref))
        excess = float(np.max(np.abs(got - ref) - bound))
        assert excess <= 0.0, (j, excess)
        return float(np.max(np.abs(got - ref) / np.maximum(bound, 1e-300)))
    err = gemm.rel_error(got, ref)
    assert err <= 1e-2, (j, err)
    return err


@pytest.mark.parametrize("flags", [0, BF16P])
def test_normal_inputs_within_tolerance(flags):
    say(f"[case] gemm_rs normal W=8 m=1024 K=512 N=768 flags={flags}, dirty signals")
    a, bt = synthgen.make_gemm_rs_inputs(m=1024, K=512, N=768)
    outs, sigs = run_gemm_rs(a, bt, flags, dirty_signals=True)
    ref = gemm.gemm_rs_ref(a, bt)
    rows = np.arange(1024 // 8)
    for j in range(8):
        check_outputs(a, bt, outs, flags, j, rows, ref[j])
        assert (sigs[j] == 1).all()


@pytest.mark.parametrize("flags", [0, BF16P])
def test_full_workload_sampled_rows(flags):
    wl = synthgen.GEMM_RS
    say(f"[case] gemm_rs full {wl.name} flags={flags} (sampled rows)")
    a, bt = synthgen.make_gemm_rs_inputs(wl)
    outs, sigs = run_gemm_rs(a, bt, flags)
    mj = wl.m // wl.W
    rng = np.random.default_rng(0)
    for j in range(wl.W):
        rows = np.unique(np.concatenate([rng.integers(0, mj, 12), [0, 255, 256, mj - 1]]))
        ref = gemm.gemm_rs_rows_ref(a, bt, j, rows)
        err = check_outputs(a, bt, outs, flags, j, rows, ref)
        say(f"[full] rank {j} error measure {err:.3e}")
        assert (sigs[j] == 1).all()


@pytest.mark.parametrize("flags", [0, BF16P])
def test_full_workload_integer_whole_output(flags):
    """The workload's shape with inputs in {-1, 0, 1}: every fp32 accumulation and
    sum is an exact integer (|value| <= 8 * 896), so the whole of every out_j
    equals the oracle's fp64 sum rounded to bf16, bit for bit."""
    wl = synthgen.GEMM_RS
    say(f"[case] gemm_rs full {wl.name} integer flags={flags} (whole output)")
    a, bt = synthgen.make_gemm_rs_inputs(wl, integer=True)
    outs, sigs = run_gemm_rs(a, bt, flags)
    ref = gemm.gemm_rs_ref(a, bt, round_partials=bool(flags & BF16P))
    for j in range(wl.W):
        np.testing.assert_array_equal(outs[j], gemm.f64_to_bf16_rne_bits(ref[j]), err_msg=f"rank {j}")
        assert (sigs[j] == 1).all()
