"""GPU parity of the AllGather + GEMM (through the C ABI) against the fp64 oracle.

* The gathered matrix G must equal the stacked shards bit for bit.
* Integer inputs in {-1, 0, 1}: every partial sum is an integer below 2^24, so
  fp32 accumulation is exact and C must equal the oracle's product rounded to
  bf16 (nearest even) bit for bit.
* Normal inputs: max relative error <= 1e-2 with the floor 0.01 * RMS(ref)
  (oracle/gemm.py ``rel_error``).
* Final signals: every tile signal 1, every part counter its tile's part count.
"""
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import moe_all2all_combine_amd as ra2a  # noqa: E402
import synthgen  # noqa: E402
from oracle import gemm  # noqa: E402

from combine_harness import say  # noqa: E402

pytestmark = pytest.mark.gpu


def parts_per_tile(m_local, K, tile_rows):
    """The library's split of a tile into AllGather parts of about 128 KiB."""
    tr = min(tile_rows, m_local)
    ntiles = math.ceil(m_local / tr)
    np0 = max(1, math.ceil(tr * K * 2 / (128 << 10)))
    rpp = math.ceil(tr / np0)
    rows_last = m_local - (ntiles - 1) * tr
    return [math.ceil(tr / rpp)] * (ntiles - 1) + [math.ceil(rows_last / rpp)]


def run_ag_gemm(shards, b, tile_rows, rank=0, flags=0, entry=None, g_pad=0):
    """b is B (K x N), or B^T (N x K) when flags has AG_B_TRANSPOSED.  `entry`:
    the binding function to call (ra2a.ag_gemm by default); g_pad: bytes of
    padding before G in its slice (an offset that is not a multiple of 128)."""
    entry = entry or ra2a.ag_gemm
    W = len(shards)
    m_local, K = shards[0].shape
    N = b.shape[0] if flags & ra2a.AG_B_TRANSPOSED else b.shape[1]
    nt, nc, nq = ra2a.ag_gemm_signal_slots(W, m_local, tile_rows)
    nsig = nt + nc + nq
    shard_bytes = m_local * K * 2
    heap = ra2a.SymmHeap(W, shard_bytes + W * shard_bytes + nsig * 128 + (1 << 16))
    try:
        off_a = heap.alloc(shard_bytes)
        if g_pad:
            heap.alloc(g_pad, 16)
        off_g = heap.alloc(W * shard_bytes, 16)
        off_s = heap.alloc(nsig * 128)
        for w in range(W):
            heap.view(off_a, (m_local, K), torch.int16, w).copy_(
                torch.from_numpy(shards[w].view(np.int16)))
        heap.view(off_g, (W * m_local, K), torch.int16, rank).fill_(0x7FC1)  # NaN poison
        bt = torch.from_numpy(b.view(np.int16)).cuda()
        ct = torch.full((W * m_local, N), 0x7FC1, dtype=torch.int16, device="cuda")
        torch.cuda.synchronize()
        entry(heap.ptr(off_a), heap.ptr(off_g), bt.data_ptr(), ct.data_ptr(),
              heap.ptr(off_s), W, rank, m_local, K, N, tile_rows, flags,
              torch.cuda.current_stream())
        torch.cuda.synchronize()
        rc = ra2a.check(heap.handle)
        assert rc == ra2a.OK, ra2a.last_error()
        g = heap.view(off_g, (W * m_local, K), torch.int16, rank).cpu().numpy().view(np.uint16)
        sig = heap.view(off_s, (nsig, ra2a.SIG_STRIDE_U64), torch.int64, rank)[:, 0].cpu().numpy()
        return ct.cpu().numpy().view(np.uint16), g, sig, (nt, nc)
    finally:
        heap.close()


def check_common(shards, b, tile_rows, c, g, sig, counts):
    m_local, K = shards[0].shape
    W = len(shards)
    np.testing.assert_array_equal(g, gemm.allgather_rows(shards))
    nt, nc = counts
    assert (sig[:nt] == 1).all(), sig[:nt]
    want_parts = np.tile(np.array(parts_per_tile(m_local, K, tile_rows)), W)
    np.testing.assert_array_equal(sig[nt:nt + nc], want_parts)


EXACT = [
    # W, m_local, K, N, tile_rows, rank
    (8, 256, 512, 512, 128, 0),
    (3, 300, 72, 200, 100, 1),     # ragged rows, columns and k
    (1, 5, 8, 8, 1, 0),            # W = 1, one-row tiles
    (16, 129, 264, 264, 64, 7),    # more shards than XCDs
    (2, 520, 1032, 776, 1000, 1),  # a tile larger than a shard
    (8, 64, 4096, 8, 512, 3),      # N smaller than one column tile
    (2, 96, 192, 136, 48, 1),      # three 64-k stages: the one refill of the ring
    (4, 64, 128, 64, 32, 2),       # two whole stages, no refill
    (2, 601, 8, 40, 128, 0),       # shard starts off the 128-byte grid: device-wide sync
    (3, 601, 72, 64, 128, 1),
]


@pytest.mark.parametrize("W,m_local,K,N,tile_rows,rank", EXACT)
def test_integer_inputs_bit_exact(W, m_local, K, N, tile_rows, rank):
    say(f"[case] ag_gemm integer W={W} m={m_local} K={K} N={N} tile={tile_rows} rank={rank}")
    shards, b = synthgen.make_integer_ag_gemm_inputs(W, m_local, K, N, seed=W + m_local)
    c, g, sig, counts = run_ag_gemm(shards, b, tile_rows, rank)
    check_common(shards, b, tile_rows, c, g, sig, counts)
    ref = gemm.ag_gemm_ref(shards, b)
    np.testing.assert_array_equal(c, gemm.f64_to_bf16_rne_bits(ref))


@pytest.mark.parametrize("flags", [0, ra2a.AG_AGENT_SYNC])
def test_normal_inputs_within_tolerance(flags):
    wl = synthgen.AG_GEMM
    say(f"[case] ag_gemm normal W=8 m=512 K=1024 N=768 flags={flags}")
    shards, b = synthgen.make_ag_gemm_inputs(wl, m_local=512, K=1024, N=768)
    c, g, sig, counts = run_ag_gemm(shards, b, 128, 0, flags)
    check_common(shards, b, 128, c, g, sig, counts)
    ref = gemm.ag_gemm_ref(shards, b)
    err = gemm.rel_error(gemm.bf16_bits_to_f64(c), ref)
    assert err <= 1e-2, err


def test_pre_transposed_b_matches():
    """Passing B^T (N x K) with AG_B_TRANSPOSED gives the same bits as passing B."""
    wl = synthgen.AG_GEMM
    say("[case] ag_gemm B vs pre-transposed B^T, W=4 m=384 K=520 N=392")
    shards, b = synthgen.make_ag_gemm_inputs(wl, m_local=384, K=520, N=392, W=4)
    c0, g0, sig0, counts = run_ag_gemm(shards, b, 128, 2, 0)
    c1, g1, sig1, _ = run_ag_gemm(shards, np.ascontiguousarray(b.T), 128, 2, ra2a.AG_B_TRANSPOSED)
    check_common(shards, b, 128, c1, g1, sig1, counts)
    np.testing.assert_array_equal(c0, c1)
    err = gemm.rel_error(gemm.bf16_bits_to_f64(c1), gemm.ag_gemm_ref(shards, b))
    assert err <= 1e-2, err


def test_full_workload_sampled_rows():
    wl = synthgen.AG_GEMM
    say("[case] ag_gemm full W=8 m=1024 K=7168 N=4096 (sampled rows)")
    shards, b = synthgen.make_ag_gemm_inputs(wl)
    c, g, sig, counts = run_ag_gemm(shards, b, wl.tile_rows, 0)
    check_common(shards, b, wl.tile_rows, c, g, sig, counts)
    rng = np.random.default_rng(0)
    M = wl.W * wl.m_local
    rows = np.unique(np.concatenate([rng.integers(0, M, 40), [0, 127, 128, 255, 256, 1023, 1024,
                                                             M - 1]]))
    ref = gemm.ag_gemm_rows_ref(shards, b, rows)
    err = gemm.rel_error(gemm.bf16_bits_to_f64(c[rows]), ref)
    say(f"[full] rel error {err:.3e}")
    assert err <= 1e-2, err


@pytest.mark.parametrize("g_pad", [16, 48])
def test_gathered_matrix_off_the_line_grid(g_pad):
    """G starting 16 or 48 bytes past a 128-byte line: row blocks share lines with
    their neighbours, so the launch synchronises device-wide; bit-exact."""
    W, m_local, K, N = 4, 520, 64, 96
    say(f"[case] ag_gemm G offset by {g_pad} bytes")
    shards, b = synthgen.make_integer_ag_gemm_inputs(W, m_local, K, N, seed=17)
    c, g, sig, counts = run_ag_gemm(shards, b, 128, 1, 0, g_pad=g_pad)
    check_common(shards, b, 128, c, g, sig, counts)
    np.testing.assert_array_equal(c, gemm.f64_to_bf16_rne_bits(gemm.ag_gemm_ref(shards, b)))


def test_full_workload_integer_inputs_bit_exact():
    """The AllGather+GEMM workload's full shape (W=8 shards of 1024 x 7168, B 7168 x
    4096) with integer inputs in {-1, 0, 1}: every output element bit for bit."""
    wl = synthgen.AG_GEMM
    say("[case] ag_gemm full shape, integer inputs, whole output")
    shards, b = synthgen.make_integer_ag_gemm_inputs(wl.W, wl.m_local, wl.K, wl.N, seed=23)
    c, g, sig, counts = run_ag_gemm(shards, b, wl.tile_rows, 0)
    check_common(shards, b, wl.tile_rows, c, g, sig, counts)
    say("[full] fp64 reference")
    ref = gemm.ag_gemm_ref(shards, b)
    np.testing.assert_array_equal(c, gemm.f64_to_bf16_rne_bits(ref))
