"""CPU oracle of the variable-size AllToAll (push) -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg use
this module; the GPU path never imports it.

Followed passage: the HyperParallel RFC, section 十, "AllToAll (Push mode)": the
ranks first exchange their receive offsets as metadata (with an all-to-all of
the split sizes), then every rank pushes each destination its segment, and a
destination's signal accumulates to the world size before it waits no longer.

Reading taken (the page gives no formula): the operation is the split-size
all-to-all of the frameworks.  Rank r's input is a sequence of rows cut, in
destination order, into W consecutive segments of send_counts[r][j] rows; rank
j's output is the concatenation, in source order r = 0 .. W-1, of the segments
addressed to it, and its receive counts are recv_counts[j][r] =
send_counts[r][j].  Rows are opaque bytes.  Rows of the input beyond the sum
of its send counts are not sent.
"""
from __future__ import annotations

from typing import List, Sequence, Tuple

import numpy as np


def _check(ins: Sequence[np.ndarray], send_counts: np.ndarray) -> Tuple[int, np.ndarray]:
    W = len(ins)
    c = np.asarray(send_counts, dtype=np.int64)
    if c.shape != (W, W):
        raise ValueError("send_counts must be W x W")
    if (c < 0).any():
        raise ValueError("negative send count")
    for r in range(W):
        if ins[r].ndim != 2:
            raise ValueError("each input is (rows, row_bytes)")
        if c[r].sum() > ins[r].shape[0]:
            raise ValueError(f"rank {r} sends more rows than it holds")
    return W, c


def send_offsets(send_counts: np.ndarray) -> np.ndarray:
    """send_off[r][j]: first input row of rank r's segment for j (exclusive prefix
    sum over destinations)."""
    c = np.asarray(send_counts, dtype=np.int64)
    return np.cumsum(c, axis=1) - c


def receive_offsets(send_counts: np.ndarray) -> np.ndarray:
    """recv_off[j][r]: first output row of rank j that source r fills (exclusive
    prefix sum over sources of the counts addressed to j) -- the metadata each
    destination hands its senders."""
    c = np.asarray(send_counts, dtype=np.int64)
    ct = c.T  # ct[j][r] = rows r sends to j
    return np.cumsum(ct, axis=1) - ct


def alltoallv(ins: Sequence[np.ndarray], send_counts: np.ndarray
              ) -> Tuple[List[np.ndarray], np.ndarray]:
    """(outs, recv_counts): outs[j] = concat_r ins[r][send segment r->j], rows of
    bytes; recv_counts[j][r] = send_counts[r][j]."""
    W, c = _check(ins, send_counts)
    so = send_offsets(c)
    outs = []
    for j in range(W):
        parts = [ins[r][so[r, j]:so[r, j] + c[r, j]] for r in range(W)]
        outs.append(np.concatenate(parts, axis=0) if parts else np.zeros((0, ins[0].shape[1]), np.uint8))
    return outs, c.T.copy()
