"""Host-side checks of the C ABI that need no GPU: exported symbols, heap
registry and symm_at arithmetic on an attached (never dereferenced) address
range, tiling queries, and argument validation before any device work."""
import ctypes
import os
import re

import pytest

import moe_all2all_combine_amd as ra2a
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ra2a.h")
FAKE_BASE = 0x7E0000000000  # host-side bookkeeping only: never dereferenced here


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ra2a_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_function_is_exported():
    names = declared_functions()
    assert len(names) >= 20
    L = ra2a.lib()
    for n in names:
        assert hasattr(L, n), f"{n} declared in include/ra2a.h but not exported"


def test_version():
    assert ra2a.version() >= 100


@pytest.fixture
def fake_heap():
    h = ra2a.symm_heap_attach(FAKE_BASE, 4, 4 << 20)
    yield h
    ra2a.symm_heap_destroy(h)


def test_symm_at_matches_oracle(fake_heap):
    base, stride, world = ra2a.symm_heap_info(fake_heap)
    assert (base, stride, world) == (FAKE_BASE, 4 << 20, 4)
    for off in (0, 8, 1234, stride - 1):
        for k in range(world):
            p = base + k * stride + off
            for r in range(-1, world + 1):
                want = oracle.symm_at(base, stride, world, p, r)
                got = ra2a.symm_at(fake_heap, p, r)
                assert got == want, (off, k, r)
    assert ra2a.symm_at(fake_heap, base - 1, 0) is None
    assert ra2a.symm_at(fake_heap, base + world * stride, 0) is None
    assert ra2a.lib().ra2a_symm_heap_find(base + 3 * stride + 5) == fake_heap
    assert ra2a.lib().ra2a_symm_heap_find(base + 4 * stride) is None


def test_symm_malloc_bump_and_exhaustion(fake_heap):
    a = ra2a.symm_malloc(fake_heap, 100)
    b = ra2a.symm_malloc(fake_heap, 10, 4096)
    assert a == 0 and b == 4096
    # default alignment: 256 B below 4 KiB, 4 KiB from 4 KiB on
    c = ra2a.symm_malloc(fake_heap, 100)
    d = ra2a.symm_malloc(fake_heap, 8192)
    e2 = ra2a.symm_malloc(fake_heap, 100, 16)
    assert (c, d, e2) == (4096 + 256, 8192, 16384)
    with pytest.raises(ra2a.Ra2aError) as e:
        ra2a.symm_malloc(fake_heap, 4 << 20)
    assert e.value.code == ra2a.ENOMEM
    with pytest.raises(ra2a.Ra2aError) as e:
        ra2a.symm_malloc(fake_heap, 8, 3)
    assert e.value.code == ra2a.EINVAL


def test_attach_rejects_overlap_and_misalignment(fake_heap):
    for args in [(FAKE_BASE + (4 << 20), 1, 4 << 20), (FAKE_BASE + 1, 1, 256), (FAKE_BASE, 0, 256),
                 (FAKE_BASE + (64 << 20), 1, 100)]:
        with pytest.raises(ra2a.Ra2aError) as e:
            ra2a.symm_heap_attach(*args)
        assert e.value.code == ra2a.EINVAL


def test_signal_slots_and_workspace():
    Q = ra2a.QUEUE_SLOTS + ra2a.RESET_FLAGS  # control words: queue words, then reset flags
    # 64-token x 1-head x 128 tiles, ADD: one slot per (S-block, head) per slice
    # the default on this shape (a source's run of a token row is 4 KiB, at most
    # 8 KiB): row units; the run is a whole 4 KiB round and 512 KiB units still
    # number 256, so 16 tokens per unit; one arrival counter per S-block in region B
    a, b, q = ra2a.rev_all2all_signal_slots(8, 512, 16, 128, "bf16")
    assert (a, b, q) == (8 * 16, 8, Q)
    p = ra2a.rev_all2all_plan(8, 512, 16, 128, "bf16")
    assert (p.mode, p.unit_rows, p.work_items) == (ra2a.MODE_ROWS, 16, 8 * 4 * 8)
    # 256 KiB units: runs shorter than a round (2 KiB), or too few 512 KiB units (128)
    p = ra2a.rev_all2all_plan(8, 1024, 8, 128, "bf16")
    assert (p.mode, p.unit_rows, p.work_items) == (ra2a.MODE_ROWS, 16, 16 * 4 * 8)
    p = ra2a.rev_all2all_plan(4, 1024, 16, 128, "bf16")
    assert (p.mode, p.unit_rows, p.work_items) == (ra2a.MODE_ROWS, 16, 16 * 4 * 4)
    # 8 KiB runs: 512 KiB units (8 tokens), 256 of them
    p = ra2a.rev_all2all_plan(8, 256, 32, 128, "bf16")
    assert (p.mode, p.unit_rows, p.work_items) == (ra2a.MODE_ROWS, 8, 4 * 8 * 8)
    # runs above 8 KiB, runs that neither divide nor are a multiple of 4 KiB (3 and
    # 6 KiB), a delayed straggler source: per-source pieces; the dispatch follows
    # the same run rule
    assert ra2a.rev_all2all_plan(8, 256, 1, 7168, "bf16").mode == ra2a.MODE_DIRECT
    assert ra2a.rev_all2all_plan(8, 512, 16, 96, "bf16").mode == ra2a.MODE_DIRECT
    assert ra2a.rev_all2all_plan(8, 512, 24, 128, "bf16").mode == ra2a.MODE_DIRECT
    assert ra2a.rev_all2all_plan(8, 512, 4, 64, "bf16").mode == ra2a.MODE_ROWS  # 512 B runs
    assert ra2a.rev_all2all_plan(8, 512, 16, 128, "bf16",
                                 ra2a.Opts(direction=ra2a.DIR_DISPATCH)).mode == ra2a.MODE_ROWS
    assert ra2a.rev_all2all_plan(8, 256, 1, 7168, "bf16",
                                 ra2a.Opts(direction=ra2a.DIR_DISPATCH)).mode == ra2a.MODE_DIRECT
    assert ra2a.rev_all2all_plan(8, 512, 16, 128, "bf16",
                                 ra2a.Opts(straggler_rank=2, straggler_delay=100)).mode == ra2a.MODE_DIRECT
    assert ra2a.rev_all2all_plan(8, 512, 16, 128, "bf16",
                                 ra2a.Opts(straggler_rank=2)).mode == ra2a.MODE_ROWS
    # per-source pieces: 16 heads merged into 4 KiB runs, so a piece (one source's 64
    # tokens) is 256 KiB and moves as two parts of 32 tokens: one arrival counter per
    # moved tile (S-block) in region B
    direct = ra2a.Opts(mode=ra2a.MODE_DIRECT)
    a, b, q = ra2a.rev_all2all_signal_slots(8, 512, 16, 128, "bf16", direct)
    assert (a, b, q) == (8 * 16, 8, Q)
    p = ra2a.rev_all2all_plan(8, 512, 16, 128, "bf16", direct)
    assert (p.mode, p.head_merge, p.piece_rows, p.pieces_per_tile) == (ra2a.MODE_DIRECT, 16, 32, 2)
    # with heads merged 8 at a time (2 KiB runs) a piece is 128 KiB, one part
    a, b, q = ra2a.rev_all2all_signal_slots(8, 512, 16, 128, "bf16", ra2a.Opts(head_merge=8))
    assert (a, b, q) == (8 * 16, 0, Q)
    # row units: region B holds one arrival counter per S-block
    a, b, q = ra2a.rev_all2all_signal_slots(8, 512, 16, 128, "bf16", ra2a.Opts(mode=ra2a.MODE_ROWS))
    assert (a, b, q) == (8 * 16, 8, Q)
    # pieces of 16 tokens: 4 per tile and source, so one arrival counter per moved tile
    # (S-block, merged head block of 8)
    a, b, q = ra2a.rev_all2all_signal_slots(8, 512, 16, 128, "bf16", ra2a.Opts(piece_rows=16, head_merge=8))
    assert (a, b, q) == (8 * 16, 8 * 2, Q)
    # staged: ring of 8 = every S-block; 256-B heads would merge 16 at a time into
    # 4 KiB runs, but that leaves only 512 pieces, so 8 at a time (1024 pieces):
    # 2 moved streams per destination
    staged = ra2a.Opts(mode=ra2a.MODE_STAGED)
    a, b, q = ra2a.rev_all2all_signal_slots(8, 512, 16, 128, "bf16", staged)
    assert (a, b, q) == (8 * 16, 8 * 2, Q)
    a, b, _ = ra2a.rev_all2all_signal_slots(8, 512, 16, 128, "bf16",
                                            ra2a.Opts(head_merge=1, ring=2, mode=ra2a.MODE_STAGED))
    assert (a, b) == (8 * 16, 2 * 16)
    # SET: one per (S-block, head, source)
    opts = ra2a.Opts(protocol=ra2a.PROTO_SET, head_merge=1, mode=ra2a.MODE_STAGED)
    a, b, _ = ra2a.rev_all2all_signal_slots(16, 2048, 32, 128, "f32", opts)
    assert (a, b) == (32 * 32 * 16, 8 * 32 * 16)
    opts = ra2a.Opts(protocol=ra2a.PROTO_SET, mode=ra2a.MODE_STAGED)  # 512-B heads merge 8 at a time
    a, b, _ = ra2a.rev_all2all_signal_slots(16, 2048, 32, 128, "f32", opts)
    assert (a, b) == (32 * 32 * 16, 8 * 4 * 16)
    # 32 x 7168 tiles: 128 S-blocks
    a, b, _ = ra2a.rev_all2all_signal_slots(8, 4096, 1, 7168, "bf16",
                                            ra2a.Opts(tile_s=32, mode=ra2a.MODE_STAGED))
    assert (a, b) == (128, 8)
    # 448 KiB of one source per tile: four pieces of 8 tokens, a counter per tile
    a, b, _ = ra2a.rev_all2all_signal_slots(8, 4096, 1, 7168, "bf16", ra2a.Opts(tile_s=32))
    assert (a, b) == (128, 128)
    a, b, _ = ra2a.rev_all2all_signal_slots(8, 4096, 1, 7168, "bf16",
                                            ra2a.Opts(tile_s=32, piece_rows=32))
    assert (a, b) == (128, 0)
    pl = ra2a.rev_all2all_plan(8, 4096, 1, 7168, "bf16", ra2a.Opts(tile_s=32))
    assert (pl.mode, pl.piece_rows, pl.pieces_per_tile, pl.work_items) == (
        ra2a.MODE_DIRECT, 8, 4, 8 * 128 * 4 * 8)
    # ragged: S=37 in tiles of 16 -> 3 blocks; D=40 in tiles of 16 -> 3 d blocks
    a, b, _ = ra2a.rev_all2all_signal_slots(3, 37, 2, 40, "bf16",
                                            ra2a.Opts(tile_s=16, tile_d=16, mode=ra2a.MODE_STAGED))
    assert (a, b) == (3 * 2 * 3, 3 * 2 * 3)  # tiles narrower than D: heads are not merged
    assert ra2a.rev_all2all_signal_slots(3, 0, 2, 40, "bf16") == (0, 0, 0)
    assert ra2a.rev_all2all_workspace_bytes(8, 512, 16, 128, "bf16") == 0  # direct: no ring
    ring = ra2a.rev_all2all_workspace_bytes(8, 512, 16, 128, "bf16", staged)
    assert ring == 8 * 64 * 16 * 8 * 128 * 2
    assert ra2a.rev_all2all_workspace_bytes(8, 512, 16, 128, "bf16", two_phase=True) == \
        512 * 8 * 16 * 128 * 2


@pytest.mark.parametrize("bad", [
    dict(W=0), dict(S=-1), dict(dtype=99), dict(inp=FAKE_BASE - 4096), dict(W=3),
    dict(out=FAKE_BASE + 1024), dict(out=FAKE_BASE + (4 << 20) - 1024), dict(out=0x1000),
    dict(signals=FAKE_BASE + 3004), dict(signals=FAKE_BASE + 1024), dict(signals=FAKE_BASE + (4 << 20) - 128),
])
def test_combine_validation(fake_heap, bad):
    args = dict(inp=FAKE_BASE, out=FAKE_BASE + (1 << 20), signals=FAKE_BASE + (2 << 20), W=4, S=8,
                H=2, D=16, dtype="bf16")
    args.update(bad)
    with pytest.raises(ra2a.Ra2aError) as e:
        ra2a.rev_all2all(args["inp"], args["out"], args["signals"], args["W"], args["S"],
                         args["H"], args["D"], args["dtype"])
    assert e.value.code == ra2a.EINVAL, e.value


def test_combine_valid_arguments_pass_validation(fake_heap):
    """With no GPU, valid arguments get past every host check and fail only at HIP."""
    try:
        import torch
        if torch.cuda.is_available():
            pytest.skip("a GPU is present; this checks the no-GPU path")
    except ImportError:
        pass
    with pytest.raises(ra2a.Ra2aError) as e:
        ra2a.rev_all2all(FAKE_BASE, FAKE_BASE + (1 << 20), FAKE_BASE + (2 << 20), 4, 8, 2, 16,
                         "bf16")
    assert e.value.code == ra2a.EHIP


def test_empty_combine_is_a_noop(fake_heap):
    ra2a.rev_all2all(FAKE_BASE, FAKE_BASE + (1 << 20), FAKE_BASE + (2 << 20), 4, 0, 2, 16, "bf16")
    ra2a.rev_all2all_two_phase(FAKE_BASE, FAKE_BASE + (1 << 20), None, 4, 5, 0, 16, "bf16")


def test_primitive_validation(fake_heap):
    L = ra2a.lib()
    assert L.ra2a_put(None, FAKE_BASE, FAKE_BASE, 8, 0, None) == ra2a.EINVAL
    assert L.ra2a_put(fake_heap, FAKE_BASE, 0x1000, 8, 4, None) == ra2a.EINVAL  # rank
    assert L.ra2a_put(fake_heap, FAKE_BASE + (4 << 20) - 4, 0x1000, 8, 0, None) == ra2a.EINVAL
    assert L.ra2a_put_with_signal(fake_heap, FAKE_BASE, 0x1000, 8, FAKE_BASE + 4, 1, 0, 0,
                                  None) == ra2a.EINVAL  # unaligned signal
    assert L.ra2a_put_with_signal(fake_heap, FAKE_BASE, 0x1000, 8, FAKE_BASE + 4096, 1, 7, 0,
                                  None) == ra2a.EINVAL  # bad op
    assert L.ra2a_wait_signal(fake_heap, FAKE_BASE, 1, 6, None) == ra2a.EINVAL
    assert L.ra2a_wait_signal(fake_heap, 0x1000, 1, 0, None) == ra2a.EINVAL
    assert L.ra2a_signal_reset(fake_heap, FAKE_BASE + (4 << 20) - 128, 2, None) == ra2a.EINVAL
    assert L.ra2a_symm_heap_create(0, 1, ctypes.byref(ctypes.c_void_p())) == ra2a.EINVAL
    assert ra2a.last_error() != ""


def test_opts_layout_matches_the_header(tmp_path):
    """The ctypes mirror of ra2a_opts_t has the C struct's size and field offsets."""
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    fields = [f[0] for f in ra2a.Opts._fields_]
    src = ["#include <stdio.h>", "#include <stddef.h>", '#include "ra2a.h"', "int main(void) {",
           '  printf("%zu\\n", sizeof(ra2a_opts_t));']
    src += [f'  printf("%zu\\n", offsetof(ra2a_opts_t, {f}));' for f in fields]
    src += ["  return 0;", "}"]
    c = tmp_path / "layout.c"
    c.write_text("\n".join(src) + "\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(root, "include"), str(c), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], check=True, capture_output=True,
                                          text=True).stdout.split()]
    assert got[0] == ctypes.sizeof(ra2a.Opts)
    assert got[1:] == [getattr(ra2a.Opts, f).offset for f in fields]


def test_dispatch_signal_slots():
    """One slot per (signal tile, source) in every slice.  By default the dispatch
    runs row units here (4 KiB runs): one arrival counter per S-block of the
    slice's own rows in region B.  With per-source pieces it merges all 16 heads
    into 4 KiB runs, so a piece (64 tokens) is 256 KiB and moves as two parts of
    32 tokens: one arrival counter per (S-block, source) in region B."""
    o = ra2a.Opts(direction=ra2a.DIR_DISPATCH)
    assert ra2a.rev_all2all_signal_slots(8, 512, 16, 128, "bf16", o) == (
        8 * 16 * 8, 8, ra2a.QUEUE_SLOTS + ra2a.RESET_FLAGS)
    assert ra2a.rev_all2all_plan(8, 512, 16, 128, "bf16", o).mode == ra2a.MODE_ROWS
    o = ra2a.Opts(direction=ra2a.DIR_DISPATCH, mode=ra2a.MODE_DIRECT)
    assert ra2a.rev_all2all_signal_slots(8, 512, 16, 128, "bf16", o) == (
        8 * 16 * 8, 8 * 8, ra2a.QUEUE_SLOTS + ra2a.RESET_FLAGS)
    p = ra2a.rev_all2all_plan(8, 512, 16, 128, "bf16", o)
    assert (p.piece_rows, p.pieces_per_tile) == (32, 2)
    # with heads kept in 2 KiB runs the pieces are 128 KiB, one part each
    o = ra2a.Opts(direction=ra2a.DIR_DISPATCH, head_merge=8)
    assert ra2a.rev_all2all_signal_slots(8, 512, 16, 128, "bf16", o) == (
        8 * 16 * 8, 0, ra2a.QUEUE_SLOTS + ra2a.RESET_FLAGS)


# ---- argument checks of the AllToAll and GEMM+ReduceScatter entry points ----------
# (all rejected before any device call, on an attached address range never dereferenced)

def _a2v(h, inp, cnt, out, rc, sig, W=4, row_bytes=64, in_rows=100, out_rows=100, chunk=0, flags=0):
    return ra2a.lib().ra2a_alltoallv(inp, cnt, out, rc, sig, W, row_bytes, in_rows, out_rows, chunk,
                                     flags, None)


def test_alltoallv_rejects_bad_arguments(fake_heap):
    b = FAKE_BASE
    inp, out, cnt, rc, sig = b, b + (1 << 20), b + (2 << 20), b + (2 << 20) + 256, b + (3 << 20)
    E = ra2a.EINVAL
    assert _a2v(fake_heap, 0x1000, cnt, out, rc, sig) == E                      # in outside any heap
    assert _a2v(fake_heap, inp, cnt, out, rc, 0x1000) == E                      # signals outside
    assert _a2v(fake_heap, inp, cnt, out, rc, sig, W=3) == E                    # W != slices
    assert _a2v(fake_heap, inp, cnt, out, rc, sig, W=33) == E                   # W above 32
    assert _a2v(fake_heap, inp + 8, cnt, out, rc, sig) == E                     # in not 16-aligned
    assert _a2v(fake_heap, inp, cnt + 4, out, rc, sig) == E                     # counts not 8-aligned
    assert _a2v(fake_heap, inp, cnt, inp + 4096, rc, sig) == E                  # out overlaps in
    assert _a2v(fake_heap, inp, cnt, out, rc, sig, out_rows=1 << 20) == E       # out past the slice
    assert _a2v(fake_heap, inp, cnt, out, rc, sig, chunk=24) == E               # chunk not 16-multiple
    assert _a2v(fake_heap, inp, cnt, out, rc, sig, flags=2) == E                # unknown flag
    assert _a2v(fake_heap, inp, cnt, out, rc, sig, row_bytes=0) == E
    assert _a2v(fake_heap, 0, cnt, out, rc, sig) == E                           # NULL


def _grs(h, x1, x2t, p, out, sig, W=4, m=64, K=64, N=64, flags=0):
    return ra2a.lib().ra2a_gemm_rs(x1, x2t, p, out, sig, W, m, K, N, flags, None)


def test_gemm_rs_rejects_bad_arguments(fake_heap):
    b = FAKE_BASE
    x1, x2t, p, out, sig = b, b + (1 << 18), b + (1 << 19), b + (1 << 20), b + (2 << 20)
    E = ra2a.EINVAL
    assert _grs(fake_heap, 0x1000, x2t, p, out, sig) == E                        # x1 outside the heap
    assert _grs(fake_heap, x1, x2t, p, out, sig, W=2) == E                       # W != slices
    assert _grs(fake_heap, x1, x2t, p, out, sig, m=66) == E                      # m not divisible by W
    assert _grs(fake_heap, x1, x2t, p, out, sig, K=12) == E                      # K not a multiple of 8
    assert _grs(fake_heap, x1, x2t, p + 8, out, sig) == E                        # partial not 16-aligned
    assert _grs(fake_heap, x1, x1 + 4096, p, out, sig) == E                      # x2t overlaps x1
    assert _grs(fake_heap, x1, x2t, p, out, b + (4 << 20) - 64) == E             # signals past the slice
    assert _grs(fake_heap, x1, x2t, p, out, sig, flags=8) == E                   # unknown flag
    assert _grs(fake_heap, x1, x2t, 0, out, sig) == E                            # NULL


def test_exit_hook_closes_open_heaps():
    """A process that exits with attached heaps open ends normally: the binding
    tracks them and its exit hook destroys them (no GPU involved: an attached
    heap that never ran makes no HIP call)."""
    import subprocess
    import sys
    import os
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = ("import sys; sys.path.insert(0, %r)\n"
            "import moe_all2all_combine_amd as ra2a\n"
            "h = ra2a.symm_heap_attach(0x7f0000000000, 2, 1 << 20)\n"
            "assert h in ra2a._open_handles\n"
            "ra2a._close_all_heaps()\n"
            "assert not ra2a._open_handles\n"
            "h2 = ra2a.symm_heap_attach(0x7f0000000000, 2, 1 << 20)\n"
            "print('ok', flush=True)\n") % root
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and "ok" in r.stdout, r.stderr
