"""Host checks of the variable-size AllToAll (no GPU): the kernel's own queue
decode, run in queue order by the library's emulator, moves exactly the oracle's
rows, every wait points backwards, the signals end where the protocol says (the
count and arrival signals at W, as the page's accumulation to the world size),
and bad counts and overflowing destinations are reported, not waited on."""
import numpy as np
import pytest

import moe_all2all_combine_amd as ra2a
import synthgen
from oracle import alltoallv as a2av

ERR_COUNTS, ERR_OVERFLOW = 2, 4

CASES = [
    # W, rows per rank, row_bytes, chunk, empty pairs
    (1, 5, 16, 0, 0),
    (2, 9, 16, 16, 1),
    (3, 40, 12, 48, 2),       # 4-byte vectors
    (4, 33, 7, 16, 3),        # 1-byte vectors, chunks not aligned to rows
    (8, 200, 64, 1024, 5),
    (8, 64, 14336, 0, 0),     # MoE rows, default chunk
    (16, 50, 32, 96, 10),
    (32, 12, 16, 32, 40),     # the largest W
]


def chunks(rows, row_bytes, chunk):
    chunk = chunk or 44 << 10
    b = rows * row_bytes
    return max(1, -(-b // chunk))


@pytest.mark.parametrize("W,rows,rb,chunk,empty", CASES)
def test_emulated_alltoallv_matches_oracle(W, rows, rb, chunk, empty):
    c = synthgen.make_alltoallv_counts(W, rows, seed=W + rows, empty_pairs=empty)
    ins = [np.random.default_rng(r).integers(0, 256, size=(rows, rb), dtype=np.uint8) for r in range(W)]
    want, want_rc = a2av.alltoallv(ins, c)
    out_rows = max(x.shape[0] for x in want) + 3
    outs, rc, sig, err, tasks = ra2a.debug_alltoallv_emulate(ins, c, out_rows, chunk)
    assert err == 0
    nc = sum(chunks(c[r, j], rb, chunk) for r in range(W) for j in range(W))
    assert tasks == 3 * W + nc
    roff = a2av.receive_offsets(c)
    for j in range(W):
        n = want[j].shape[0]
        np.testing.assert_array_equal(outs[j][:n], want[j])
        assert not outs[j][n:].any(), "rows past the received ones are untouched"
        np.testing.assert_array_equal(rc[j, :W], want_rc[j])
        assert rc[j, W] == n
        assert sig[j, 0] == W and sig[j, 1 + 2 * W] == W  # count and arrival signals
        for r in range(W):
            assert sig[r, 1 + j] == roff[j, r] + 1        # offset handed to sender r
            assert sig[j, 1 + W + r] == chunks(c[r, j], rb, chunk)
    assert sig[0, 2 + 2 * W] == tasks


def test_bad_counts_send_nothing_and_are_reported():
    W, rows, rb = 4, 20, 16
    c = synthgen.make_alltoallv_counts(W, rows, seed=1)
    ins = [np.full((rows, rb), r + 1, dtype=np.uint8) for r in range(W)]
    bad = c.copy()
    bad[1, 2] = -3          # a negative count
    bad[3, 0] += 1          # more rows than rank 3 holds
    outs, rc, sig, err, _ = ra2a.debug_alltoallv_emulate(ins, bad, 4 * rows)
    assert err & ERR_COUNTS and not err & ERR_OVERFLOW
    usable = c.copy()
    usable[1] = 0
    usable[3] = 0
    want, want_rc = a2av.alltoallv(ins, usable)
    for j in range(W):
        np.testing.assert_array_equal(outs[j][:want[j].shape[0]], want[j])
        np.testing.assert_array_equal(rc[j, :W], want_rc[j])
        assert sig[j, 0] == W and sig[j, 1 + 2 * W] == W


def test_overflowing_destination_is_reported_and_skipped():
    W, rows, rb = 3, 30, 16
    c = np.array([[10, 10, 10], [5, 20, 5], [10, 10, 10]])
    ins = [np.full((rows, rb), r + 1, dtype=np.uint8) for r in range(W)]
    outs, rc, sig, err, _ = ra2a.debug_alltoallv_emulate(ins, c, 38)  # rank 1 receives 40 rows
    assert err == ERR_OVERFLOW
    want, _ = a2av.alltoallv(ins, c)
    np.testing.assert_array_equal(outs[0][:25], want[0])
    np.testing.assert_array_equal(outs[2][:25], want[2])
    # rank 1: sources 0 and 1 fit (rows 0..29), source 2's rows 30..39 would not
    np.testing.assert_array_equal(outs[1][:30], want[1][:30])
    assert not outs[1][30:].any()
    assert all(sig[j, 1 + 2 * W] == W for j in range(W)), "every signal still completes"


def test_signal_slots_and_argument_checks():
    assert ra2a.alltoallv_signal_slots(8) == 19
    for W in (0, 33):
        with pytest.raises(ra2a.Ra2aError) as e:
            ra2a.alltoallv_signal_slots(W)
        assert e.value.code == ra2a.EINVAL
    ins = [np.zeros((4, 16), np.uint8)] * 2
    for chunk in (8, 24, -16):
        with pytest.raises(ra2a.Ra2aError):
            ra2a.debug_alltoallv_emulate(ins, np.ones((2, 2)), 8, chunk)
