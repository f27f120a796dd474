"""MI355X-native Reverse All2All (EP-MoE combine) over a symmetric heap.

Thin Python binding of ``libra2a.so`` (C ABI declared in ``include/ra2a.h``):
argument marshalling only -- every step of every operation runs in the
library's HIP kernels for gfx950.  PyTorch provides device memory (the heap
can be a torch allocation) and streams.  There is no fallback: if the library
is not built, importing a function raises.

Functions keep the C names without the ``ra2a_`` prefix.  Failures raise
``Ra2aError`` carrying the library's status code and message.
"""
from __future__ import annotations

import atexit
import ctypes
import os
import weakref
from typing import Optional, Sequence, Tuple

__all__ = [
    "Ra2aError", "Opts", "SymmHeap", "lib", "OK", "EINVAL", "ENOMEM", "EHIP", "ETIMEOUT",
    "EUNSUPPORTED", "EDATA", "A2V_SKIP_RESET", "alltoallv_signal_slots", "alltoallv", "debug_alltoallv_emulate", "SIG_SET", "SIG_ADD", "PROTO_ADD", "PROTO_SET", "MODE_DIRECT", "MODE_STAGED",
    "QUEUE_SLOTS", "RS_AGENT_SYNC", "RS_SKIP_RESET", "RS_BF16_PARTIALS", "gemm_rs_sizes", "gemm_rs", "debug_gemm_rs_plan", "MODE_BULK", "MODE_PULL", "MODE_ROWS", "DIR_COMBINE", "DIR_DISPATCH", "all2all_dispatch", "all2all_dispatch_ex", "RESET_FLAGS", "CMP_EQ", "CMP_NE", "CMP_GT", "CMP_GE", "CMP_LT",
    "CMP_LE", "SIG_STRIDE_BYTES", "DTYPES", "symm_heap_create", "symm_heap_attach",
    "symm_heap_destroy", "symm_malloc", "symm_heap_info", "symm_at", "put", "get",
    "put_with_signal", "signal_op", "wait_signal", "signal_reset", "rev_all2all",
    "rev_all2all_ex", "rev_all2all_two_phase", "rev_all2all_plan", "Plan", "rev_all2all_signal_slots",
    "rev_all2all_workspace_bytes", "check", "last_error", "version", "ag_gemm",
    "ag_gemm_signal_slots", "ag_gemm_noalloc", "debug_ag_gemm_plan", "AG_AGENT_SYNC", "AG_SKIP_RESET",
    "AG_B_TRANSPOSED",
]

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libra2a.so")

OK, EINVAL, ENOMEM, EHIP, ETIMEOUT, EUNSUPPORTED, EDATA = 0, -1, -2, -3, -4, -5, -6
SIG_SET, SIG_ADD = 0, 1
PROTO_ADD, PROTO_SET = 1, 2
MODE_DIRECT, MODE_STAGED = 1, 2
MODE_BULK = 3
MODE_PULL = 4
MODE_ROWS = 5
QUEUE_SLOTS = 18
DIR_COMBINE = 0
DIR_DISPATCH = 1
RESET_FLAGS = 64
AG_AGENT_SYNC, AG_SKIP_RESET, AG_B_TRANSPOSED = 1, 2, 4
CMP_EQ, CMP_NE, CMP_GT, CMP_GE, CMP_LT, CMP_LE = range(6)
SIG_STRIDE_BYTES = 128
SIG_STRIDE_U64 = 16
# element type name -> (ABI code, bytes)
DTYPES = {"u8": (0, 1), "bf16": (1, 2), "f16": (2, 2), "i32": (3, 4), "f32": (4, 4),
          "i64": (5, 8), "f64": (6, 8)}


class Ra2aError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"ra2a error {code}: {msg}")
        self.code = code


class Opts(ctypes.Structure):
    """Mirror of ``ra2a_opts_t``."""

    _fields_ = [
        ("tile_s", ctypes.c_int64), ("tile_h", ctypes.c_int64), ("tile_d", ctypes.c_int64),
        ("protocol", ctypes.c_int32), ("ring", ctypes.c_int32), ("wg_per_cu", ctypes.c_int32),
        ("lookahead", ctypes.c_int32), ("straggler_rank", ctypes.c_int32),
        ("straggler_delay", ctypes.c_uint32), ("straggler_seed", ctypes.c_uint64),
        ("timestamps", ctypes.c_void_p), ("mode", ctypes.c_int32),
        ("consumer_split", ctypes.c_int32), ("skip_reset", ctypes.c_int32),
        ("stream_batch", ctypes.c_int32), ("agent_sync", ctypes.c_int32),
        ("head_merge", ctypes.c_int32), ("separate_reset", ctypes.c_int32),
        ("direction", ctypes.c_int32), ("unit_rows", ctypes.c_int32),
        ("piece_rows", ctypes.c_int32), ("reserved", ctypes.c_int32 * 1),
    ]

    def __init__(self, **kw):
        super().__init__()
        self.straggler_rank = -1
        self.protocol = PROTO_ADD
        for k, v in kw.items():
            if v is not None:
                setattr(self, k, v)


_lib = None


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                          "(hipcc --offload-arch=gfx950); there is no fallback path")
    L = ctypes.CDLL(LIB_PATH)
    vp, sz, i32, i64, u64 = (ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int64,
                             ctypes.c_uint64)
    pp = ctypes.POINTER(ctypes.c_void_p)
    sig = {
        "ra2a_symm_heap_create": (i32, [i32, sz, pp]),
        "ra2a_symm_heap_attach": (i32, [vp, i32, sz, pp]),
        "ra2a_symm_heap_destroy": (i32, [vp]),
        "ra2a_symm_malloc": (i32, [vp, sz, sz, ctypes.POINTER(sz)]),
        "ra2a_symm_heap_info": (i32, [vp, pp, ctypes.POINTER(sz), ctypes.POINTER(i32)]),
        "ra2a_symm_heap_find": (vp, [vp]),
        "ra2a_symm_at": (vp, [vp, vp, i32]),
        "ra2a_symm_heap_set_spin_timeout": (i32, [vp, u64]),
        "ra2a_put_with_signal": (i32, [vp, vp, vp, sz, vp, u64, i32, i32, vp]),
        "ra2a_put": (i32, [vp, vp, vp, sz, i32, vp]),
        "ra2a_get": (i32, [vp, vp, vp, sz, i32, vp]),
        "ra2a_signal_op": (i32, [vp, vp, u64, i32, i32, vp]),
        "ra2a_wait_signal": (i32, [vp, vp, u64, i32, vp]),
        "ra2a_signal_reset": (i32, [vp, vp, i64, vp]),
        "ra2a_rev_all2all_signal_slots": (i32, [i32, i64, i64, i64, i32, vp, ctypes.POINTER(i64),
                                                ctypes.POINTER(i64), ctypes.POINTER(i64)]),
        "ra2a_rev_all2all_plan": (i32, [i32, i64, i64, i64, i32, vp, vp]),
        "ra2a_rev_all2all_workspace_bytes": (i32, [i32, i64, i64, i64, i32, vp, i32,
                                                   ctypes.POINTER(sz)]),
        "ra2a_rev_all2all": (i32, [vp, vp, vp, i32, i64, i64, i64, i32, vp]),
        "ra2a_rev_all2all_ex": (i32, [vp, vp, vp, i32, i64, i64, i64, i32, vp, vp]),
        "ra2a_rev_all2all_two_phase": (i32, [vp, vp, vp, i32, i64, i64, i64, i32, vp]),
        "ra2a_all2all_dispatch": (i32, [vp, vp, vp, i32, i64, i64, i64, i32, vp]),
        "ra2a_all2all_dispatch_ex": (i32, [vp, vp, vp, i32, i64, i64, i64, i32, vp, vp]),
        "ra2a_check": (i32, [vp]),
        "ra2a_ag_gemm_signal_slots": (i32, [i32, i64, i32, ctypes.POINTER(i64), ctypes.POINTER(i64),
                                            ctypes.POINTER(i64)]),
        "ra2a_ag_gemm": (i32, [vp, vp, vp, vp, vp, i32, i32, i64, i64, i64, i32, i32, vp]),
        "ra2a_ag_gemm_noalloc": (i32, [vp, vp, vp, vp, vp, i32, i32, i64, i64, i64, i32, i32, vp]),
        "ra2a_debug_ag_gemm_plan": (i32, [i32, i32, i64, i64, i64, i32, i32, ctypes.POINTER(i64)]),
        "ra2a_gemm_rs_sizes": (i32, [i32, i64, i64, i64, i32, ctypes.POINTER(i64),
                                     ctypes.POINTER(i64), ctypes.POINTER(sz)]),
        "ra2a_gemm_rs": (i32, [vp, vp, vp, vp, vp, i32, i64, i64, i64, i32, vp]),
        "ra2a_debug_gemm_rs_plan": (i32, [i32, i64, i64, i64, i32, ctypes.POINTER(i64)]),
        "ra2a_alltoallv_signal_slots": (i32, [i32, ctypes.POINTER(i64)]),
        "ra2a_alltoallv": (i32, [vp, vp, vp, vp, vp, i32, i64, i64, i64, i64, i32, vp]),
        "ra2a_debug_alltoallv_emulate": (i32, [i32, i64, i64, i64, i64, ctypes.POINTER(vp),
                                               ctypes.POINTER(i64), ctypes.POINTER(vp),
                                               ctypes.POINTER(i64), ctypes.POINTER(ctypes.c_uint64),
                                               ctypes.POINTER(ctypes.c_uint32), ctypes.POINTER(i64)]),
        "ra2a_debug_emulate_pipelined": (i32, [ctypes.POINTER(vp), ctypes.POINTER(vp),
                                               ctypes.POINTER(vp), i32, i64, i64, i64, i32, vp,
                                               i32, i32]),
        "ra2a_last_error": (ctypes.c_char_p, []),
        "ra2a_version": (i32, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def last_error() -> str:
    return lib().ra2a_last_error().decode()


def version() -> int:
    return lib().ra2a_version()


def _ok(rc: int) -> None:
    if rc != OK:
        raise Ra2aError(rc, last_error())


def _stream(stream) -> Optional[int]:
    """hipStream_t handle from a torch stream, an int handle or None (default stream)."""
    if stream is None:
        return None
    if hasattr(stream, "cuda_stream"):
        return stream.cuda_stream or None
    return int(stream) or None


def _dtype(dtype) -> int:
    if isinstance(dtype, int):
        return dtype
    return DTYPES[dtype][0]


def _opts(opts):
    if opts is None:
        return None
    if isinstance(opts, dict):
        opts = Opts(**opts)
    return ctypes.byref(opts)


# ---- heap -------------------------------------------------------------------

# Heaps still open when the interpreter exits are closed by an atexit hook,
# while torch and the HIP runtime are intact.  (Left to object finalizers or to
# the library's own unload, their device synchronize and frees would run in
# whatever order the process tears down torch, the runtime and a profiler.)
# The hook is registered again when the first torch-backed heap is made, after
# torch is imported, so that it runs before torch's own exit handlers (atexit
# runs handlers last-registered first).
_open_handles = set()
_torch_heaps = weakref.WeakSet()
_hook_after_torch = False


def _close_all_heaps() -> None:
    for h in list(_torch_heaps):
        try:
            h.close()
        except Exception:
            pass
    for handle in list(_open_handles):
        try:
            symm_heap_destroy(handle)
        except Exception:
            _open_handles.discard(handle)


atexit.register(_close_all_heaps)


def symm_heap_create(world: int, slice_bytes: int) -> int:
    h = ctypes.c_void_p()
    _ok(lib().ra2a_symm_heap_create(world, slice_bytes, ctypes.byref(h)))
    _open_handles.add(h.value)
    return h.value


def symm_heap_attach(base: int, world: int, stride: int) -> int:
    h = ctypes.c_void_p()
    _ok(lib().ra2a_symm_heap_attach(base, world, stride, ctypes.byref(h)))
    _open_handles.add(h.value)
    return h.value


def symm_heap_destroy(heap: int) -> None:
    _open_handles.discard(heap)
    _ok(lib().ra2a_symm_heap_destroy(heap))


def symm_malloc(heap: int, nbytes: int, align: int = 0) -> int:
    off = ctypes.c_size_t()
    _ok(lib().ra2a_symm_malloc(heap, nbytes, align, ctypes.byref(off)))
    return off.value


def symm_heap_info(heap: int) -> Tuple[int, int, int]:
    base = ctypes.c_void_p()
    stride = ctypes.c_size_t()
    world = ctypes.c_int()
    _ok(lib().ra2a_symm_heap_info(heap, ctypes.byref(base), ctypes.byref(stride),
                                  ctypes.byref(world)))
    return base.value, stride.value, world.value


def symm_at(heap: int, ptr: int, rank: int) -> Optional[int]:
    return lib().ra2a_symm_at(heap, ptr, rank)


def set_spin_timeout(heap: int, timeout_us: int) -> None:
    _ok(lib().ra2a_symm_heap_set_spin_timeout(heap, timeout_us))


# ---- primitives ---------------------------------------------------------------

def put(heap: int, dst_sym: int, src: int, nbytes: int, target_rank: int, stream=None) -> None:
    _ok(lib().ra2a_put(heap, dst_sym, src, nbytes, target_rank, _stream(stream)))


def get(heap: int, dst: int, src_sym: int, nbytes: int, source_rank: int, stream=None) -> None:
    _ok(lib().ra2a_get(heap, dst, src_sym, nbytes, source_rank, _stream(stream)))


def put_with_signal(heap: int, dst_sym: int, src: int, nbytes: int, sig_sym: int, value: int,
                    sig_op: int, target_rank: int, stream=None) -> None:
    _ok(lib().ra2a_put_with_signal(heap, dst_sym, src, nbytes, sig_sym, value, sig_op,
                                   target_rank, _stream(stream)))


def signal_op(heap: int, sig_sym: int, value: int, sig_op: int, target_rank: int,
              stream=None) -> None:
    _ok(lib().ra2a_signal_op(heap, sig_sym, value, sig_op, target_rank, _stream(stream)))


def wait_signal(heap: int, sig: int, cmp_value: int, cmp_op: int, stream=None) -> None:
    _ok(lib().ra2a_wait_signal(heap, sig, cmp_value, cmp_op, _stream(stream)))


def signal_reset(heap: int, sig_sym: int, n_slots: int, stream=None) -> None:
    _ok(lib().ra2a_signal_reset(heap, sig_sym, n_slots, _stream(stream)))


def check(heap: int) -> int:
    """Status of the heap's device-side checks (RA2A_OK, RA2A_ETIMEOUT or RA2A_EDATA), without raising."""
    return lib().ra2a_check(heap)


# ---- combine ------------------------------------------------------------------

def rev_all2all_signal_slots(W: int, S: int, H: int, D: int, dtype,
                             opts=None) -> Tuple[int, int, int]:
    """(data signals, hand-back counters, work-queue words) per slice."""
    a = ctypes.c_int64()
    b = ctypes.c_int64()
    c = ctypes.c_int64()
    _ok(lib().ra2a_rev_all2all_signal_slots(W, S, H, D, _dtype(dtype), _opts(opts),
                                            ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)))
    return a.value, b.value, c.value


class Plan(ctypes.Structure):
    """Mirror of ``ra2a_plan_t``: what a combine with given options resolves to."""

    _fields_ = [
        ("mode", ctypes.c_int32), ("protocol", ctypes.c_int32),
        ("tile_s", ctypes.c_int64), ("tile_h", ctypes.c_int64), ("tile_d", ctypes.c_int64),
        ("head_merge", ctypes.c_int32), ("piece_rows", ctypes.c_int32),
        ("pieces_per_tile", ctypes.c_int32), ("unit_rows", ctypes.c_int32),
        ("tile_slots", ctypes.c_int64), ("credit_slots", ctypes.c_int64),
        ("queue_slots", ctypes.c_int64), ("work_items", ctypes.c_int64),
        ("workspace_bytes", ctypes.c_size_t),
    ]


def rev_all2all_plan(W: int, S: int, H: int, D: int, dtype, opts=None) -> Plan:
    pl = Plan()
    _ok(lib().ra2a_rev_all2all_plan(W, S, H, D, _dtype(dtype), _opts(opts), ctypes.byref(pl)))
    return pl


def rev_all2all_workspace_bytes(W: int, S: int, H: int, D: int, dtype, opts=None,
                                two_phase: bool = False) -> int:
    n = ctypes.c_size_t()
    _ok(lib().ra2a_rev_all2all_workspace_bytes(W, S, H, D, _dtype(dtype), _opts(opts),
                                               int(two_phase), ctypes.byref(n)))
    return n.value


def rev_all2all(inp: int, out: int, signals: int, W: int, S: int, H: int, D: int, dtype,
                stream=None) -> None:
    _ok(lib().ra2a_rev_all2all(inp, out, signals, W, S, H, D, _dtype(dtype), _stream(stream)))


def rev_all2all_ex(inp: int, out: int, signals: int, W: int, S: int, H: int, D: int, dtype,
                   opts=None, stream=None) -> None:
    _ok(lib().ra2a_rev_all2all_ex(inp, out, signals, W, S, H, D, _dtype(dtype), _opts(opts),
                                  _stream(stream)))


def all2all_dispatch(inp: int, out: int, signals: int, W: int, S: int, H: int, D: int, dtype,
                     stream=None) -> None:
    """Forward All2All: out_r[j*S+s, h, d] = in_j[s, r*H+h, d] (the combine's inverse)."""
    _ok(lib().ra2a_all2all_dispatch(inp, out, signals, W, S, H, D, _dtype(dtype),
                                    _stream(stream)))


def all2all_dispatch_ex(inp: int, out: int, signals: int, W: int, S: int, H: int, D: int, dtype,
                        opts=None, stream=None) -> None:
    _ok(lib().ra2a_all2all_dispatch_ex(inp, out, signals, W, S, H, D, _dtype(dtype), _opts(opts),
                                       _stream(stream)))


def rev_all2all_two_phase(inp: int, out: int, signals: Optional[int], W: int, S: int, H: int,
                          D: int, dtype, stream=None) -> None:
    _ok(lib().ra2a_rev_all2all_two_phase(inp, out, signals, W, S, H, D, _dtype(dtype),
                                         _stream(stream)))


def debug_emulate_pipelined(inputs, W: int, S: int, H: int, D: int, dtype, opts=None,
                            num_cus: int = 256, blocks_per_cu: int = 2):
    """Host emulation of the pipelined kernel's address arithmetic (no GPU).

    ``inputs``: W C-contiguous numpy arrays of S*W*H*D elements.  Returns
    (outputs, signals): W output arrays shaped (S, H*W, D) and W uint64 arrays of
    final signal values (data signals, ring hand-back counters, queue words).
    """
    import numpy as np
    n_tile, n_credit, n_queue = rev_all2all_signal_slots(W, S, H, D, dtype, opts)
    outs = [np.empty((S, H * W, D), dtype=inputs[0].dtype) for _ in range(W)]
    sigs = [np.zeros(n_tile + n_credit + n_queue, dtype=np.uint64) for _ in range(W)]
    vp = ctypes.c_void_p
    pin = (vp * W)(*[a.ctypes.data for a in inputs])
    pout = (vp * W)(*[a.ctypes.data for a in outs])
    psig = (vp * W)(*[a.ctypes.data for a in sigs])
    _ok(lib().ra2a_debug_emulate_pipelined(pin, pout, psig, W, S, H, D, _dtype(dtype),
                                           _opts(opts), num_cus, blocks_per_cu))
    return outs, sigs


# ---- AllGather + GEMM -----------------------------------------------------------

def ag_gemm_signal_slots(W: int, m_local: int, tile_rows: int) -> Tuple[int, int, int]:
    """(tile signals, part counters, queue words) in the gathering rank's slice."""
    a, b, c = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    _ok(lib().ra2a_ag_gemm_signal_slots(W, m_local, tile_rows, ctypes.byref(a), ctypes.byref(b),
                                        ctypes.byref(c)))
    return a.value, b.value, c.value


def ag_gemm(a_shards: int, gathered: int, b: int, c: int, signals: int, W: int, rank: int,
            m_local: int, K: int, N: int, tile_rows: int = 128, flags: int = 0, stream=None) -> None:
    _ok(lib().ra2a_ag_gemm(a_shards, gathered, b, c, signals, W, rank, m_local, K, N, tile_rows,
                           flags, _stream(stream)))


def ag_gemm_noalloc(a_shards: int, gathered: int, b: int, c: int, signals: int, W: int, rank: int,
                    m_local: int, K: int, N: int, tile_rows: int = 128, flags: int = 0,
                    stream=None) -> None:
    """ra2a_ag_gemm_noalloc: the AllGather+GEMM without any device allocation."""
    _ok(lib().ra2a_ag_gemm_noalloc(a_shards, gathered, b, c, signals, W, rank, m_local, K, N,
                                   tile_rows, flags, _stream(stream)))


def debug_ag_gemm_plan(W: int, rank: int, m_local: int, K: int, N: int, tile_rows: int,
                       num_xcd: int = 8) -> int:
    """Host check of the AllGather+GEMM work queues; returns the queue length per group."""
    n = ctypes.c_int64()
    _ok(lib().ra2a_debug_ag_gemm_plan(W, rank, m_local, K, N, tile_rows, num_xcd, ctypes.byref(n)))
    return n.value


# ---- torch-backed heap --------------------------------------------------------

class SymmHeap:
    """A symmetric heap whose memory is one torch allocation on the current GPU.

    ``world`` slices of ``stride`` bytes (rounded up to 2 MiB); slice r is
    simulated rank r's heap.  ``alloc`` reserves the same offset in every
    slice; ``view`` returns a torch tensor over one slice's copy of a buffer.
    """

    def __init__(self, world: int, slice_bytes: int, device=None):
        import torch
        global _hook_after_torch
        if not _hook_after_torch:  # see _close_all_heaps
            atexit.register(_close_all_heaps)
            _hook_after_torch = True
        align = 2 << 20
        self.world = world
        self.stride = (slice_bytes + align - 1) // align * align
        self.mem = torch.empty(world * self.stride + 256, dtype=torch.uint8,
                               device=device or "cuda")
        raw = self.mem.data_ptr()
        self.pad = (-raw) % 256
        self.base = raw + self.pad
        self.handle = symm_heap_attach(self.base, world, self.stride)
        _torch_heaps.add(self)

    def alloc(self, nbytes: int, align: int = 0) -> int:
        return symm_malloc(self.handle, nbytes, align)

    def ptr(self, offset: int, rank: int = 0) -> int:
        return self.base + rank * self.stride + offset

    def view(self, offset: int, shape: Sequence[int], dtype, rank: int = 0):
        import torch
        n = 1
        for s in shape:
            n *= s
        nbytes = n * torch.empty((), dtype=dtype).element_size()
        start = self.pad + rank * self.stride + offset
        return self.mem[start:start + nbytes].view(dtype).view(*shape)

    def close(self) -> None:
        """Destroy the heap handle, then drop the torch memory it lived in."""
        if self.handle:
            symm_heap_destroy(self.handle)
            self.handle = None
        self.mem = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ---- GEMM + ReduceScatter --------------------------------------------------------

RS_AGENT_SYNC = 1
RS_SKIP_RESET = 2
RS_BF16_PARTIALS = 4


def gemm_rs_sizes(W: int, m: int, K: int, N: int, flags: int = 0) -> Tuple[int, int, int]:
    """(tile signal slots, queue words, receive-area bytes) per slice."""
    a, b, c = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_size_t()
    _ok(lib().ra2a_gemm_rs_sizes(W, m, K, N, flags, ctypes.byref(a), ctypes.byref(b),
                                 ctypes.byref(c)))
    return a.value, b.value, c.value


def gemm_rs(x1: int, x2t: int, partial: int, out: int, signals: int, W: int, m: int, K: int,
            N: int, flags: int = 0, stream=None) -> None:
    """out_j = rows [j*m/W, (j+1)*m/W) of sum_r x1_r @ x2_r (x2 passed transposed)."""
    _ok(lib().ra2a_gemm_rs(x1, x2t, partial, out, signals, W, m, K, N, flags, _stream(stream)))


def debug_gemm_rs_plan(W: int, m: int, K: int, N: int, num_xcd: int = 8) -> int:
    n = ctypes.c_int64()
    _ok(lib().ra2a_debug_gemm_rs_plan(W, m, K, N, num_xcd, ctypes.byref(n)))
    return n.value


# ---- variable-size AllToAll -------------------------------------------------------

A2V_SKIP_RESET = 1


def alltoallv_signal_slots(W: int) -> int:
    n = ctypes.c_int64()
    _ok(lib().ra2a_alltoallv_signal_slots(W, ctypes.byref(n)))
    return n.value


def alltoallv(inp: int, send_counts: int, out: int, recv_counts: int, signals: int, W: int,
              row_bytes: int, in_rows: int, out_rows: int, chunk_bytes: int = 0, flags: int = 0,
              stream=None) -> None:
    """Split-size all-to-all of rows: out_j = concat over r of rank r's segment for j."""
    _ok(lib().ra2a_alltoallv(inp, send_counts, out, recv_counts, signals, W, row_bytes, in_rows,
                             out_rows, chunk_bytes, flags, _stream(stream)))


def debug_alltoallv_emulate(ins, send_counts, out_rows: int, chunk_bytes: int = 0):
    """Host emulation of the AllToAll's queue: (outs, recv_counts, signals, error bits, tasks).

    ins: W uint8 arrays (in_rows, row_bytes); send_counts: W x W integers."""
    import numpy as np
    W = len(ins)
    in_rows, row_bytes = ins[0].shape
    ins = [np.ascontiguousarray(x, dtype=np.uint8) for x in ins]
    outs = [np.zeros((out_rows, row_bytes), dtype=np.uint8) for _ in range(W)]
    cnt = np.ascontiguousarray(np.asarray(send_counts, dtype=np.int64).reshape(W, W))
    rc = np.zeros((W, W + 1), dtype=np.int64)
    sig = np.zeros((W, 2 * W + 3), dtype=np.uint64)
    err = ctypes.c_uint32()
    tasks = ctypes.c_int64()
    ip = (ctypes.c_void_p * W)(*[x.ctypes.data for x in ins])
    op = (ctypes.c_void_p * W)(*[x.ctypes.data for x in outs])
    _ok(lib().ra2a_debug_alltoallv_emulate(
        W, row_bytes, in_rows, out_rows, chunk_bytes, ip,
        cnt.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), op,
        rc.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
        sig.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)), ctypes.byref(err), ctypes.byref(tasks)))
    return outs, rc, sig, err.value, tasks.value
