"""CPU oracle for the Reverse All2All combine, its signal protocol and the AllGather+GEMM.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or execute anything here.  The
GPU path (``moe_all2all_combine_amd``) shares no code with this package and
never imports it; this package never imports the GPU path.

Contents and the passages they follow:

* ``combine`` / ``combine_dest`` (C, ``combine.c``): the plain definition
  out_j[s, r*H+h, d] = in_r[j*S+s, h, d] of "Reverse All2All (EP MoE
  Distributed Kernel)", section "Reverse All2All Operator Semantics", with the
  column order r*H + h and the row split j*S + s taken from the same page's
  MTE listing ("Triton-Distributed Reverse All2All Operator").
* ``dispatch`` / ``dispatch_dest`` (C, ``combine.c``): the forward All2All read
  as the combine's inverse, out_r[j*S+s, h, d] = in_j[s, r*H+h, d] (same page,
  sections "Reverse All2All Operator Semantics" and "EP MoE Scenario").
* ``source_of``: the same definition read backwards, for one output element.
* ``symm_at``: "Distributed Architecture Design", section 5.3: the symmetric
  offset of a pointer inside its own heap, added to the target's heap base.
* ``signal_apply`` / ``compare``: section 2.3 (SignalOp SET / ADD) and section
  6.3 (the six wait predicates) of the same page.
* ``protocol``: the producer/consumer signal protocol (see its docstring).
* ``gemm``: the fp64 AllGather+GEMM and GEMM+ReduceScatter.
* ``alltoallv``: the variable-size AllToAll (the HyperParallel RFC, section 十,
  "AllToAll (Push mode)"), read as the frameworks' split-size all-to-all.

Pins (what ties these to something other than themselves) live in
``tests/test_oracle_*.py`` and run with ``-m "not gpu"``.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Sequence

import numpy as np

from . import alltoallv, gemm, protocol  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "_oracle.so")
_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from .build import build
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        i64 = ctypes.c_int64
        lib.oracle_combine_dest.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p,
                                            i64, i64, i64, i64, i64, i64]
        lib.oracle_combine_dest.restype = ctypes.c_int
        lib.oracle_dispatch_dest.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p,
                                             i64, i64, i64, i64, i64, i64]
        lib.oracle_dispatch_dest.restype = ctypes.c_int
        lib.oracle_source_of.argtypes = [i64] * 8 + [ctypes.POINTER(i64)] * 3
        lib.oracle_source_of.restype = None
        lib.oracle_allgather.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p,
                                         i64, i64, i64]
        lib.oracle_allgather.restype = None
        _lib = lib
    return _lib


def _ptrs(arrays: Sequence[np.ndarray]):
    arr = (ctypes.c_void_p * len(arrays))()
    for i, a in enumerate(arrays):
        arr[i] = a.ctypes.data
    return arr


def _check_inputs(inputs: Sequence[np.ndarray]):
    W = len(inputs)
    if W < 1:
        raise ValueError("need at least one rank")
    shape = inputs[0].shape
    dt = inputs[0].dtype
    if len(shape) != 3 or shape[0] % W:
        raise ValueError(f"each input must be (S*W, H, D); got {shape} for W={W}")
    for a in inputs:
        if a.shape != shape or a.dtype != dt or not a.flags.c_contiguous:
            raise ValueError("inputs must share one shape and dtype and be C-contiguous")
    return W, shape[0] // W, shape[1], shape[2], dt


def combine_dest(inputs: Sequence[np.ndarray], j: int) -> np.ndarray:
    """out_j of shape (S, H*W, D) from the W inputs (same dtype)."""
    W, S, H, D, dt = _check_inputs(inputs)
    out = np.empty((S, H * W, D), dtype=dt)
    rc = _load().oracle_combine_dest(_ptrs(inputs), out.ctypes.data, j, W, S, H, D,
                                     dt.itemsize)
    if rc:
        raise ValueError("oracle_combine_dest rejected its arguments")
    return out


def combine_dest_rows(inputs: Sequence[np.ndarray], out_j: np.ndarray, j: int, s0: int,
                      s1: int) -> None:
    """Rows [s0, s1) of out_j (a preallocated (S, H*W, D) array), written in place.

    The definition restricted to those rows is itself a combine of the same form:
    destination 0 of a problem with S' = s1 - s0 whose sources are in_r rows
    [j*S + s0, j*S + s1), so the same C function computes it from offset pointers
    (no other arithmetic).  Lets a caller split one combine over threads by (j, s)."""
    W, S, H, D, dt = _check_inputs(inputs)
    if not (0 <= s0 <= s1 <= S) or out_j.shape != (S, H * W, D) or out_j.dtype != dt \
            or not out_j.flags.c_contiguous:
        raise ValueError("bad row range or output array")
    if s1 == s0:
        return
    e = dt.itemsize
    sub = (ctypes.c_void_p * W)(*[a.ctypes.data + (j * S + s0) * H * D * e for a in inputs])
    rc = _load().oracle_combine_dest(sub, out_j.ctypes.data + s0 * H * W * D * e, 0, W, s1 - s0,
                                     H, D, e)
    if rc:
        raise ValueError("oracle_combine_dest rejected its arguments")


def combine(inputs: Sequence[np.ndarray]) -> List[np.ndarray]:
    """All W outputs, each of shape (S, H*W, D)."""
    W = len(inputs)
    return [combine_dest(inputs, j) for j in range(W)]


def dispatch_dest(inputs: Sequence[np.ndarray], r: int) -> np.ndarray:
    """out_r of shape (S*W, H, D) from the W dispatch inputs, each (S, H*W, D)."""
    W = len(inputs)
    if W < 1:
        raise ValueError("need at least one rank")
    shape, dt = inputs[0].shape, inputs[0].dtype
    if len(shape) != 3 or shape[1] % W:
        raise ValueError(f"each dispatch input must be (S, H*W, D); got {shape} for W={W}")
    for a in inputs:
        if a.shape != shape or a.dtype != dt or not a.flags.c_contiguous:
            raise ValueError("inputs must share one shape and dtype and be C-contiguous")
    S, H, D = shape[0], shape[1] // W, shape[2]
    out = np.empty((S * W, H, D), dtype=dt)
    rc = _load().oracle_dispatch_dest(_ptrs(inputs), out.ctypes.data, r, W, S, H, D, dt.itemsize)
    if rc:
        raise ValueError("oracle_dispatch_dest rejected its arguments")
    return out


def dispatch(inputs: Sequence[np.ndarray]) -> List[np.ndarray]:
    """All W dispatch outputs, each of shape (S*W, H, D): out_r[j*S+s, h, d] = in_j[s, r*H+h, d]."""
    return [dispatch_dest(inputs, r) for r in range(len(inputs))]


def source_of(j: int, s: int, c: int, d: int, W: int, S: int, H: int, D: int):
    """(source rank, source row, source head) of out_j[s, c, d]."""
    r = ctypes.c_int64()
    row = ctypes.c_int64()
    h = ctypes.c_int64()
    _load().oracle_source_of(j, s, c, d, W, S, H, D, ctypes.byref(r), ctypes.byref(row),
                             ctypes.byref(h))
    return r.value, row.value, h.value


def allgather(shards: Sequence[np.ndarray]) -> np.ndarray:
    """Row shards stacked in rank order (byte copy, C)."""
    W = len(shards)
    m, k = shards[0].shape
    out = np.empty((W * m, k), dtype=shards[0].dtype)
    for s in shards:
        if s.shape != (m, k) or not s.flags.c_contiguous:
            raise ValueError("shards must share one shape and be C-contiguous")
    _load().oracle_allgather(_ptrs(shards), out.ctypes.data, W, m, k * out.itemsize)
    return out


def symm_at(base: int, stride: int, world: int, ptr: int, rank: int):
    """Address of ``ptr``'s symmetric twin on ``rank``; None if out of the heap or rank.

    The heap is ``world`` equal slices of ``stride`` bytes starting at ``base``;
    slice k is rank k's heap.  The pointer's symmetric offset is its distance
    from the base of the slice that holds it.
    """
    if not (0 <= rank < world) or not (base <= ptr < base + world * stride):
        return None
    own_slice = (ptr - base) // stride
    offset = ptr - (base + own_slice * stride)
    return base + rank * stride + offset


SIG_SET = "set"
SIG_ADD = "add"
CMP_OPS = ("eq", "ne", "gt", "ge", "lt", "le")


def signal_apply(old: int, value: int, op: str) -> int:
    """New signal value: SET stores ``value``; ADD adds it (64-bit unsigned wrap)."""
    if op == SIG_SET:
        return value & 0xFFFFFFFFFFFFFFFF
    if op == SIG_ADD:
        return (old + value) & 0xFFFFFFFFFFFFFFFF
    raise ValueError(op)


def compare(value: int, cmp_value: int, op: str) -> bool:
    """Whether a wait on ``op`` against ``cmp_value`` is satisfied by ``value`` (unsigned)."""
    if op == "eq":
        return value == cmp_value
    if op == "ne":
        return value != cmp_value
    if op == "gt":
        return value > cmp_value
    if op == "ge":
        return value >= cmp_value
    if op == "lt":
        return value < cmp_value
    if op == "le":
        return value <= cmp_value
    raise ValueError(op)
