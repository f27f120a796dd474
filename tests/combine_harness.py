"""GPU test harness for the combine: a torch-backed symmetric heap with in, out
and signal buffers, uploads of seeded inputs and downloads of results.  Calls
only the C ABI (through the package's ctypes binding)."""
from __future__ import annotations

import sys
from typing import List, Optional

import numpy as np
import torch

import moe_all2all_combine_amd as ra2a
import synthgen

TORCH_BITS = {1: torch.uint8, 2: torch.int16, 4: torch.int32, 8: torch.int64}


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def opts_for(wl: synthgen.CombineWorkload, **kw) -> ra2a.Opts:
    proto = ra2a.PROTO_SET if wl.protocol == synthgen.PROTOCOL_SET else ra2a.PROTO_ADD
    base = dict(tile_s=wl.tile_s, tile_h=wl.tile_h, tile_d=wl.tile_d, protocol=proto)
    base.update(kw)
    return ra2a.Opts(**base)


class CombineCase:
    """Buffers of one combine workload inside one heap."""

    def __init__(self, wl: synthgen.CombineWorkload, opts: Optional[ra2a.Opts] = None,
                 two_phase: bool = True, extra: int = 0):
        self.wl = wl
        self.opts = opts if opts is not None else opts_for(wl)
        W, S, H, D = wl.W, wl.S, wl.H, wl.D
        self.n_tile, self.n_credit, self.n_queue = ra2a.rev_all2all_signal_slots(
            W, S, H, D, wl.dtype, self.opts)
        ring = ra2a.rev_all2all_workspace_bytes(W, S, H, D, wl.dtype, self.opts)
        full = ra2a.rev_all2all_workspace_bytes(W, S, H, D, wl.dtype, None, True) if two_phase else 0
        nb = wl.bytes_per_rank
        sig_bytes = max(1, self.n_tile + self.n_credit + self.n_queue) * ra2a.SIG_STRIDE_BYTES
        slice_bytes = 2 * nb + ring + full + sig_bytes + 8 * 4096 + extra
        self.heap = ra2a.SymmHeap(W, slice_bytes)
        self.off_in = self.heap.alloc(max(nb, 1))
        self.off_out = self.heap.alloc(max(nb, 1))
        self.off_sig = self.heap.alloc(sig_bytes)
        self.bits = TORCH_BITS[wl.elem_bytes]

    # pointers (slice 0)
    @property
    def p_in(self):
        return self.heap.ptr(self.off_in)

    @property
    def p_out(self):
        return self.heap.ptr(self.off_out)

    @property
    def p_sig(self):
        return self.heap.ptr(self.off_sig)

    def in_view(self, r):
        wl = self.wl
        return self.heap.view(self.off_in, (wl.S * wl.W, wl.H, wl.D), self.bits, r)

    def out_view(self, j):
        wl = self.wl
        return self.heap.view(self.off_out, (wl.S, wl.H * wl.W, wl.D), self.bits, j)

    def upload(self, inputs: List[np.ndarray]) -> None:
        for r, a in enumerate(inputs):
            self.in_view(r).copy_(torch.from_numpy(np.ascontiguousarray(a).view(
                {1: np.uint8, 2: np.int16, 4: np.int32, 8: np.int64}[self.wl.elem_bytes])))
        torch.cuda.synchronize()

    def fill_out(self, byte: int) -> None:
        for j in range(self.wl.W):
            self.out_view(j).view(torch.uint8).fill_(byte)
        torch.cuda.synchronize()

    def download(self, j: int) -> np.ndarray:
        return self.out_view(j).cpu().numpy().view(self.wl.np_dtype)

    def signals(self, j: int) -> np.ndarray:
        n = self.n_tile + self.n_credit
        v = self.heap.view(self.off_sig, (max(n, 1), ra2a.SIG_STRIDE_U64), torch.int64, j)
        return v[:n, 0].cpu().numpy()

    def control_words(self) -> np.ndarray:
        """Slice 0's words after the data signals and hand-back counters."""
        n0 = self.n_tile + self.n_credit
        v = self.heap.view(self.off_sig, (n0 + self.n_queue, ra2a.SIG_STRIDE_U64), torch.int64, 0)
        return v[n0:, 0].cpu().numpy()

    def queue_words(self) -> np.ndarray:
        """The work-queue words of slice 0: per group (8) its claim counter and
        take-over counter, then the mask of fully claimed groups and a spare."""
        return self.control_words()[:ra2a.QUEUE_SLOTS]

    def reset_flags(self) -> np.ndarray:
        """The in-launch reset's flags (slice 0), after the work-queue words."""
        return self.control_words()[ra2a.QUEUE_SLOTS:ra2a.QUEUE_SLOTS + ra2a.RESET_FLAGS]

    def fill_signals(self, byte: int) -> None:
        """Every signal-array byte of every slice (control words included) := byte."""
        n = max(1, self.n_tile + self.n_credit + self.n_queue) * ra2a.SIG_STRIDE_BYTES
        for r in range(self.wl.W):
            self.heap.view(self.off_sig, (n,), torch.uint8, r).fill_(byte)

    def run_pipelined(self, stream=None) -> None:
        wl = self.wl
        ra2a.rev_all2all_ex(self.p_in, self.p_out, self.p_sig, wl.W, wl.S, wl.H, wl.D, wl.dtype,
                            self.opts, stream or torch.cuda.current_stream())

    def run_two_phase(self, stream=None) -> None:
        wl = self.wl
        ra2a.rev_all2all_two_phase(self.p_in, self.p_out, None, wl.W, wl.S, wl.H, wl.D, wl.dtype,
                                   stream or torch.cuda.current_stream())

    def check_device(self) -> None:
        rc = ra2a.check(self.heap.handle)
        assert rc == ra2a.OK, f"device-side wait failed: {ra2a.last_error()}"

    def close(self) -> None:
        self.heap.close()
