"""GPU parity of the GEMM + ReduceScatter (through the C ABI) against the fp64 oracle.

* Integer inputs in {-1, 0, 1}: every partial and every sum is an integer below
  2^24, exact in fp32, so out_j must equal the oracle's sum rounded to bf16
  (nearest even) bit for bit.
* Normal inputs: max relative error <= 1e-2 with the floor 0.01 * RMS(ref)
  (oracle/gemm.py ``rel_error``).
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


def run_gemm_rs(a_bits, bt_bits, flags=0, dirty_signals=False):
    W = len(a_bits)
    m, K = a_bits[0].shape
    N = bt_bits[0].shape[0]
    mj = m // W
    nt, nq, pbytes = ra2a.gemm_rs_sizes(W, m, K, N)
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
        ra2a.gemm_rs(heap.ptr(oa), heap.ptr(ob), heap.ptr(op), heap.ptr(oo), heap.ptr(osg), W, m,
                     K, N, flags, torch.cuda.current_stream())
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
    (3, 300, 72, 202),       # N not a multiple of 4: the reduce's one-column path
    (1, 5, 8, 8),            # W = 1: a plain GEMM
    (16, 16 * 130, 64, 264),  # more ranks than XCDs, ragged tiles
    (2, 2 * 520, 1032, 776),
    (5, 5 * 40, 4096, 16),   # long K, narrow N
]


@pytest.mark.parametrize("W,m,K,N", EXACT)
@pytest.mark.parametrize("flags", [0, ra2a.RS_AGENT_SYNC])
def test_integer_inputs_bit_exact(W, m, K, N, flags):
    say(f"[case] gemm_rs integer W={W} m={m} K={K} N={N} flags={flags}")
    a, bt = synthgen.make_gemm_rs_inputs(m=m, K=K, N=N, W=W, integer=True)
    outs, sigs = run_gemm_rs(a, bt, flags)
    ref = gemm.gemm_rs_ref(a, bt)
    for j in range(W):
        np.testing.assert_array_equal(outs[j], gemm.f64_to_bf16_rne_bits(ref[j]),
                                      err_msg=f"rank {j}")
        assert (sigs[j] == 1).all(), sigs[j]


def test_normal_inputs_within_tolerance():
    say("[case] gemm_rs normal W=8 m=1024 K=512 N=768, dirty signals")
    a, bt = synthgen.make_gemm_rs_inputs(m=1024, K=512, N=768)
    outs, sigs = run_gemm_rs(a, bt, 0, dirty_signals=True)
    ref = gemm.gemm_rs_ref(a, bt)
    for j in range(8):
        err = gemm.rel_error(gemm.bf16_bits_to_f64(outs[j]), ref[j])
        assert err <= 1e-2, (j, err)
        assert (sigs[j] == 1).all()


def test_full_workload_sampled_rows():
    wl = synthgen.GEMM_RS
    say(f"[case] gemm_rs full {wl.name} (sampled rows)")
    a, bt = synthgen.make_gemm_rs_inputs(wl)
    outs, sigs = run_gemm_rs(a, bt)
    mj = wl.m // wl.W
    rng = np.random.default_rng(0)
    for j in range(wl.W):
        rows = np.unique(np.concatenate([rng.integers(0, mj, 12), [0, 255, 256, mj - 1]]))
        ref = gemm.gemm_rs_rows_ref(a, bt, j, rows)
        err = gemm.rel_error(gemm.bf16_bits_to_f64(outs[j][rows]), ref)
        say(f"[full] rank {j} rel error {err:.3e}")
        assert err <= 1e-2, (j, err)
        assert (sigs[j] == 1).all()
