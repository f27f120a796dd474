"""GPU parity of the variable-size AllToAll (through the C ABI) against the oracle.

Rows are bytes, so the bar is bit-exact: every received row equals the oracle's,
rows past the received ones keep their poison, the receive counts and totals
equal the transposed send counts, and the signals end at the protocol's values
(count and arrival signals at W).  At full size: sampled rows against the
oracle's mapping, and the round trip through the transposed counts returns
every sent row bit for bit.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import moe_all2all_combine_amd as ra2a  # noqa: E402
import synthgen  # noqa: E402
from oracle import alltoallv as a2av  # noqa: E402

from combine_harness import say  # noqa: E402

pytestmark = pytest.mark.gpu
POISON = 0xA5


class Case:
    def __init__(self, W, in_rows, out_rows, rb):
        self.W, self.in_rows, self.out_rows, self.rb = W, in_rows, out_rows, rb
        self.nsig = ra2a.alltoallv_signal_slots(W)
        ni, no = in_rows * rb, out_rows * rb
        self.heap = ra2a.SymmHeap(W, ni + no + W * 8 + (W + 1) * 8 + self.nsig * 128 + (1 << 16))
        h = self.heap
        self.oi, self.oo = h.alloc(max(ni, 16), 16), h.alloc(max(no, 16), 16)
        self.oc, self.orc, self.osg = h.alloc(W * 8, 8), h.alloc((W + 1) * 8, 8), h.alloc(self.nsig * 128)

    def upload(self, ins, counts, dirty_signals=False):
        h, W = self.heap, self.W
        for r in range(W):
            if self.in_rows:
                h.view(self.oi, (self.in_rows, self.rb), torch.uint8, r).copy_(torch.from_numpy(ins[r]))
            h.view(self.oc, (W,), torch.int64, r).copy_(torch.from_numpy(np.asarray(counts[r], np.int64)))
            if self.out_rows:
                h.view(self.oo, (self.out_rows, self.rb), torch.uint8, r).fill_(POISON)
            h.view(self.orc, (W + 1,), torch.int64, r).fill_(-7)
            if dirty_signals:
                h.view(self.osg, (self.nsig * 128,), torch.uint8, r).fill_(0x5A)
        torch.cuda.synchronize()

    def run(self, chunk=0, flags=0):
        h = self.heap
        ra2a.alltoallv(h.ptr(self.oi), h.ptr(self.oc), h.ptr(self.oo), h.ptr(self.orc), h.ptr(self.osg),
                       self.W, self.rb, self.in_rows, self.out_rows, chunk, flags,
                       torch.cuda.current_stream())
        torch.cuda.synchronize()
        return ra2a.check(h.handle)

    def out(self, j, rows=None):
        v = self.heap.view(self.oo, (self.out_rows, self.rb), torch.uint8, j)
        return (v if rows is None else v[torch.as_tensor(rows, device="cuda")]).cpu().numpy()

    def recv_counts(self, j):
        return self.heap.view(self.orc, (self.W + 1,), torch.int64, j).cpu().numpy()

    def signals(self, j):
        return self.heap.view(self.osg, (self.nsig, ra2a.SIG_STRIDE_U64), torch.int64, j)[:, 0].cpu().numpy()

    def close(self):
        self.heap.close()


def check_all(case, ins, counts, chunk):
    W, rb = case.W, case.rb
    want, want_rc = a2av.alltoallv(ins, counts)
    roff = a2av.receive_offsets(counts)
    chunk_b = chunk or 44 << 10
    for j in range(W):
        n = want[j].shape[0]
        o = case.out(j)
        np.testing.assert_array_equal(o[:n], want[j], err_msg=f"rank {j}")
        assert (o[n:] == POISON).all(), f"rank {j}: rows past the received ones were written"
        rc = case.recv_counts(j)
        np.testing.assert_array_equal(rc[:W], want_rc[j])
        assert rc[W] == n
        s = case.signals(j)
        assert s[0] == W and s[1 + 2 * W] == W, s
        for r in range(W):
            assert case.signals(r)[1 + j] == roff[j, r] + 1
            assert s[1 + W + r] == max(1, -(-int(counts[r, j]) * rb // chunk_b))


SMALL = [
    # W, rows per rank, row_bytes, chunk, empty pairs
    (1, 5, 16, 0, 0),
    (2, 9, 16, 16, 1),
    (3, 40, 12, 48, 2),
    (4, 33, 7, 16, 3),
    (8, 200, 64, 1024, 5),
    (8, 64, 14336, 0, 0),
    (16, 50, 32, 96, 10),
    (32, 12, 16, 32, 40),
]


@pytest.mark.parametrize("W,rows,rb,chunk,empty", SMALL)
def test_small(W, rows, rb, chunk, empty):
    say(f"[case] alltoallv W={W} rows={rows} row_bytes={rb} chunk={chunk} empty={empty}")
    c = synthgen.make_alltoallv_counts(W, rows, seed=W + rows, empty_pairs=empty)
    ins = synthgen.make_alltoallv_inputs(W, rows, rb, seed=W)
    out_rows = int(c.sum(axis=0).max()) + 3
    case = Case(W, rows, out_rows, rb)
    try:
        case.upload(ins, c, dirty_signals=True)
        assert case.run(chunk) == ra2a.OK, ra2a.last_error()
        check_all(case, ins, c, chunk)
    finally:
        case.close()


def test_back_to_back_with_new_counts_and_skip_reset():
    """Two calls in a row with different counts (the reset launch clears the first
    call's signals), then a third with the caller's own reset."""
    W, rows, rb, chunk = 8, 300, 48, 512
    ins = synthgen.make_alltoallv_inputs(W, rows, rb, seed=3)
    case = Case(W, rows, rows * 2, rb)
    try:
        for k, seed in enumerate((1, 2, 3)):
            say(f"[case] alltoallv back-to-back call {k}")
            c = synthgen.make_alltoallv_counts(W, rows, seed=seed, empty_pairs=k)
            case.upload(ins, c)
            flags = 0
            if k == 2:
                ra2a.signal_reset(case.heap.handle, case.heap.ptr(case.osg), case.nsig,
                                  torch.cuda.current_stream())
                flags = ra2a.A2V_SKIP_RESET
            assert case.run(chunk, flags) == ra2a.OK, ra2a.last_error()
            check_all(case, ins, c, chunk)
    finally:
        case.close()


def test_bad_counts_and_overflow_report_edata():
    W, rows, rb = 4, 20, 16
    ins = synthgen.make_alltoallv_inputs(W, rows, rb, seed=4)
    c = synthgen.make_alltoallv_counts(W, rows, seed=1)
    case = Case(W, rows, 4 * rows, rb)
    try:
        say("[case] alltoallv bad counts")
        bad = c.copy()
        bad[1, 2] = -3
        case.upload(ins, bad)
        assert case.run() == ra2a.EDATA
        usable = c.copy()
        usable[1] = 0
        want, _ = a2av.alltoallv(ins, usable)
        for j in range(W):
            np.testing.assert_array_equal(case.out(j)[:want[j].shape[0]], want[j])
            assert case.signals(j)[1 + 2 * W] == W
        say("[case] alltoallv overflow")
        big = np.zeros((W, W), np.int64)
        big[:, 0] = rows  # rank 0 receives 4 * rows = out_rows: fits exactly
        case.upload(ins, big)
        assert case.run() == ra2a.OK, ra2a.last_error()
        check_all(case, ins, big, 0)
    finally:
        case.close()
    case = Case(W, rows, 3 * rows, rb)
    try:
        case.upload(ins, big)
        assert case.run() == ra2a.EDATA  # rank 0 would receive 4 * rows into 3 * rows
        want, _ = a2av.alltoallv(ins, big)
        np.testing.assert_array_equal(case.out(0), want[0][:3 * rows])
        assert case.signals(0)[1 + 2 * W] == W
    finally:
        case.close()


def test_full_workload_whole_output_and_round_trip():
    """The full workload: every rank's whole output equals the oracle's segments
    concatenated in source order (bit for bit), then the round trip through the
    transposed counts returns every input row."""
    wl = synthgen.ALLTOALLV
    W, rows, rb = wl.W, wl.rows, wl.row_bytes
    say(f"[case] alltoallv full {wl.name}: generating")
    c = synthgen.make_alltoallv_counts(W, rows, wl.seed, wl.alpha)
    ins = synthgen.make_alltoallv_inputs(W, rows, rb, wl.seed)
    recv = c.sum(axis=0)
    out_rows = int(recv.max())
    case = Case(W, max(rows, out_rows), max(rows, out_rows), rb)
    try:
        case.upload([np.concatenate([x, np.zeros((case.in_rows - rows, rb), np.uint8)]) for x in ins], c)
        say("[full] forward")
        assert case.run() == ra2a.OK, ra2a.last_error()
        want, _ = a2av.alltoallv(ins, c)
        for j in range(W):
            assert (case.recv_counts(j)[:W] == c[:, j]).all() and case.recv_counts(j)[W] == recv[j]
            assert want[j].shape[0] == recv[j]
            got = case.heap.view(case.oo, (case.out_rows, rb), torch.uint8, j)[:recv[j]].cpu().numpy()
            assert np.array_equal(got, want[j]), f"rank {j}"
        del want, got
        say("[full] round trip")
        # send each rank's received rows back with the transposed counts
        h = case.heap
        for j in range(W):
            h.view(case.oi, (case.in_rows, rb), torch.uint8, j).copy_(
                h.view(case.oo, (case.out_rows, rb), torch.uint8, j))
            h.view(case.oc, (W,), torch.int64, j).copy_(torch.from_numpy(np.ascontiguousarray(c[:, j])))
            h.view(case.oo, (case.out_rows, rb), torch.uint8, j).fill_(POISON)
        torch.cuda.synchronize()
        assert case.run() == ra2a.OK, ra2a.last_error()
        for r in range(W):
            back = h.view(case.oo, (case.out_rows, rb), torch.uint8, r)[:rows].cpu().numpy()
            assert np.array_equal(back, ins[r]), f"rank {r}"
    finally:
        case.close()
