"""The allocation-free AllGather+GEMM (ra2a_ag_gemm_noalloc, through the C ABI)
against the allocating entry point ra2a_ag_gemm: two calls in a row, the second
on a smaller problem, each bit for bit equal to ra2a_ag_gemm's output on the
same integer inputs (exact in fp32, so both also equal the fp64 oracle rounded
to bf16); B passed as is (B^T then lives in the static scratch) and
pre-transposed.  An oversized B is refused before anything runs."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import moe_all2all_combine_amd as ra2a  # noqa: E402
import synthgen  # noqa: E402
from oracle import gemm  # noqa: E402

from combine_harness import say  # noqa: E402
from test_gpu_ag_gemm import check_common, run_ag_gemm  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("transposed", [False, True])
def test_noalloc_matches_allocating_entry_point(transposed):
    flags = ra2a.AG_B_TRANSPOSED if transposed else 0
    for (W, m_local, K, N, tr, rank) in [(8, 512, 1024, 768, 128, 0), (3, 200, 136, 96, 64, 2)]:
        say(f"[case] ag_gemm_noalloc W={W} m={m_local} K={K} N={N} transposed={transposed}")
        shards, b = synthgen.make_integer_ag_gemm_inputs(W, m_local, K, N, seed=W * 7 + K)
        bb = np.ascontiguousarray(b.T) if transposed else b
        c1, g1, s1, counts = run_ag_gemm(shards, bb, tr, rank, flags, entry=ra2a.ag_gemm_noalloc)
        c0, g0, s0, _ = run_ag_gemm(shards, bb, tr, rank, flags, entry=ra2a.ag_gemm)
        check_common(shards, b, tr, c1, g1, s1, counts)
        np.testing.assert_array_equal(c1, c0)
        # tile signals and part counters (the queue words after them depend on the
        # synchronisation mode: device-wide until an allocating call has measured
        # the XCDs, which the first call in a fresh process has not)
        n = sum(counts)
        np.testing.assert_array_equal(s1[:n], s0[:n])
        np.testing.assert_array_equal(c1, gemm.f64_to_bf16_rne_bits(gemm.ag_gemm_ref(shards, b)))


def test_noalloc_refuses_oversized_b():
    W, m_local, K, N = 1, 8, 8192, 4104  # B^T of 8192 * 4104 * 2 bytes > 64 MiB
    heap = ra2a.SymmHeap(W, 4 << 20)
    try:
        oa, og, osg = heap.alloc(m_local * K * 2), heap.alloc(m_local * K * 2), heap.alloc(1 << 16)
        b = torch.zeros(K, N, dtype=torch.int16, device="cuda")
        c = torch.zeros(m_local, N, dtype=torch.int16, device="cuda")
        with pytest.raises(ra2a.Ra2aError) as e:
            ra2a.ag_gemm_noalloc(heap.ptr(oa), heap.ptr(og), b.data_ptr(), c.data_ptr(),
                                 heap.ptr(osg), W, 0, m_local, K, N, 128, 0,
                                 torch.cuda.current_stream())
        assert e.value.code == ra2a.EINVAL and "scratch" in str(e.value)
    finally:
        heap.close()
