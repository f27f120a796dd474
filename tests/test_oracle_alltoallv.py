"""Pins of the variable-size AllToAll oracle (oracle/alltoallv.py).

Pinned against: element-by-element loops on tiny shapes, torch's gloo
all_to_all_single across real CPU processes (a library routine computing the
same split-size exchange), the combine oracle (the equal-split case is the
combine's exchange phase, a layout fixed by an independently pinned oracle), the
round trip through the transposed counts, and planted mistakes.
"""
import os
import socket

import numpy as np
import pytest
import torch
import torch.distributed as dist
import torch.multiprocessing as mp

import oracle
from oracle import alltoallv as a2av
import synthgen


def _rows(W, n, row_bytes, seed):
    rng = np.random.default_rng(seed)
    return [rng.integers(0, 256, size=(n, row_bytes), dtype=np.uint8) for _ in range(W)]


def test_matches_elementwise_loops():
    W, n, rb = 3, 7, 5
    ins = _rows(W, n, rb, 0)
    c = np.array([[2, 0, 3], [1, 4, 2], [0, 0, 6]])
    outs, rc = a2av.alltoallv(ins, c)
    for j in range(W):
        want = []
        for r in range(W):
            start = 0
            for jj in range(j):
                start += c[r][jj]
            for k in range(c[r][j]):
                want.append([ins[r][start + k][b] for b in range(rb)])
        assert outs[j].tolist() == want
        assert [rc[j][r] for r in range(W)] == [c[r][j] for r in range(W)]


def test_offsets_hand_worked():
    c = np.array([[2, 0, 3], [1, 4, 2], [0, 0, 6]])
    # rank 0's segments start at rows 0, 2, 2; rank 1's at 0, 1, 5; rank 2's at 0, 0, 0
    assert a2av.send_offsets(c).tolist() == [[0, 2, 2], [0, 1, 5], [0, 0, 0]]
    # rank 0 receives 2 + 1 + 0 rows: sources start at 0, 2, 3; rank 2 receives 3 + 2 + 6
    assert a2av.receive_offsets(c).tolist() == [[0, 2, 3], [0, 0, 4], [0, 3, 5]]


def _free_port():
    s = socket.socket()
    s.bind(("127.0.0.1", 0))
    p = s.getsockname()[1]
    s.close()
    return p


def _gloo_rank(rank, W, port, ins, counts, results):
    os.environ["MASTER_ADDR"] = "127.0.0.1"
    os.environ["MASTER_PORT"] = str(port)
    dist.init_process_group("gloo", rank=rank, world_size=W)
    try:
        x = torch.from_numpy(ins[rank][:counts[rank].sum()].copy())
        recv = [int(counts[r][rank]) for r in range(W)]
        out = torch.empty((sum(recv), x.shape[1]), dtype=torch.uint8)
        dist.all_to_all_single(out, x, output_split_sizes=recv,
                               input_split_sizes=[int(v) for v in counts[rank]])
        results[rank] = out.numpy().tobytes()
    finally:
        dist.destroy_process_group()


def test_matches_gloo_all_to_all_single():
    W, n, rb = 3, 40, 12
    ins = _rows(W, n, rb, 1)
    c = synthgen.make_alltoallv_counts(W, n, seed=3, empty_pairs=2)
    want, _ = a2av.alltoallv(ins, c)
    ctx = mp.get_context("spawn")
    port = _free_port()
    with ctx.Manager() as m:
        results = m.dict()
        procs = [ctx.Process(target=_gloo_rank, args=(r, W, port, ins, c, results))
                 for r in range(W)]
        for p in procs:
            p.start()
        for p in procs:
            p.join(120)
            assert p.exitcode == 0
        for j in range(W):
            assert results[j] == want[j].tobytes(), f"rank {j}"


def test_equal_splits_are_the_combine_exchange():
    """With every count S, out_j's rows r*S + s hold in_r[j*S + s]: the combine's
    exchange layout, so out_j row r*S + s (H*D elements) is the combine output
    out_j[s, r*H:(r+1)*H, :]."""
    W, S, H, D = 3, 4, 2, 8
    wl = synthgen.small_workload(W, S, H, D, "i32", seed=5)
    ins = synthgen.make_inputs(wl)
    rows = [x.reshape(S * W, H * D).view(np.uint8).reshape(S * W, H * D * 4) for x in ins]
    outs, _ = a2av.alltoallv(rows, np.full((W, W), S))
    comb = oracle.combine(ins)
    for j in range(W):
        got = outs[j].view(np.int32).reshape(W, S, H, D)
        want = comb[j].reshape(S, W, H, D).transpose(1, 0, 2, 3)
        np.testing.assert_array_equal(got, want)


def test_round_trip_through_transposed_counts():
    W, n, rb = 4, 30, 3
    ins = _rows(W, n, rb, 2)
    c = synthgen.make_alltoallv_counts(W, n, seed=4, empty_pairs=3)
    outs, rc = a2av.alltoallv(ins, c)
    back, _ = a2av.alltoallv(outs, rc)
    for r in range(W):
        np.testing.assert_array_equal(back[r], ins[r])


def test_rows_past_the_counts_are_not_sent_and_bad_counts_rejected():
    ins = _rows(2, 10, 4, 3)
    c = np.array([[1, 2], [3, 0]])
    outs, _ = a2av.alltoallv(ins, c)
    assert outs[0].shape[0] == 4 and outs[1].shape[0] == 2
    with pytest.raises(ValueError):
        a2av.alltoallv(ins, np.array([[6, 5], [0, 0]]))
    with pytest.raises(ValueError):
        a2av.alltoallv(ins, np.array([[-1, 2], [0, 0]]))


def test_planted_mistakes_are_caught():
    W, n, rb = 3, 7, 5
    ins = _rows(W, n, rb, 6)
    c = np.array([[2, 0, 3], [1, 4, 2], [0, 0, 6]])
    ok, _ = a2av.alltoallv(ins, c)
    so = a2av.send_offsets(c)
    mutants = {
        "sources in reverse order": [np.concatenate([ins[r][so[r, j]:so[r, j] + c[r, j]]
                                                     for r in reversed(range(W))]) for j in range(W)],
        "counts transposed": [np.concatenate([ins[r][so[r, j]:so[r, j] + c[j, r]]
                                              for r in range(W)]) for j in range(W)],
        "inclusive send offsets": [np.concatenate([ins[r][so[r, j] + c[r, j]:so[r, j] + 2 * c[r, j]]
                                                   for r in range(W)]) for j in range(W)],
    }
    for name, outs in mutants.items():
        assert any(o.shape != ok[j].shape or not np.array_equal(o, ok[j]) for j, o in enumerate(outs)), name
