"""A process that exits with symmetric heaps still open (a torch-backed heap
that ran a combine, so its device error word exists, and a library-owned heap)
must end with status 0: the binding's exit hook closes them while torch and
the HIP runtime are intact."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SCRIPT = r"""
import sys
sys.path.insert(0, {root!r})
import torch
import moe_all2all_combine_amd as ra2a
W, S, H, D = 2, 8, 4, 16
nb = S * W * H * D * 4
heap = ra2a.SymmHeap(W, 4 * nb + (1 << 20))
oi, oo, osg = heap.alloc(nb), heap.alloc(nb), heap.alloc(1 << 16)
for r in range(W):
    heap.view(oi, (S * W * H * D,), torch.int32, r).copy_(
        torch.arange(S * W * H * D, dtype=torch.int32, device="cuda") + r * S * W * H * D)
ra2a.rev_all2all(heap.ptr(oi), heap.ptr(oo), heap.ptr(osg), W, S, H, D, "i32",
                 torch.cuda.current_stream())
torch.cuda.synchronize()
assert ra2a.check(heap.handle) == ra2a.OK
owned = ra2a.symm_heap_create(2, 1 << 20)
print("exiting with two open heaps", flush=True)
"""


def test_exit_with_open_heaps_returns_zero():
    r = subprocess.run([sys.executable, "-c", SCRIPT.format(root=ROOT)], capture_output=True,
                       text=True, timeout=240)
    print(r.stdout, r.stderr[-2000:])
    assert "exiting with two open heaps" in r.stdout
    assert r.returncode == 0, r.stderr[-2000:]
