"""Pins of the fp64 AllGather+GEMM oracle and its bf16 helpers.

Pinned against: fixed bit patterns of the bf16 format, torch's own float32 ->
bf16 conversion (a library routine), hand-worked ties, a brute-force triple
loop on tiny shapes and exact integer products.
"""
import numpy as np
import torch

import oracle
from oracle import gemm


def test_bf16_decode_known_patterns():
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x4049, 0x7F7F, 0x0080, 0x3C00],
                    dtype=np.uint16)
    want = [1.0, -2.0, 0.0, -0.0, 3.140625, 3.3895313892515355e38, 2.0 ** -126, 2.0 ** -7]
    got = gemm.bf16_bits_to_f64(bits)
    np.testing.assert_array_equal(got, np.array(want))
    assert np.signbit(got[3])


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 2**16, size=10000, dtype=np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]  # finite patterns
    t = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64)
    np.testing.assert_array_equal(gemm.bf16_bits_to_f64(bits), t.numpy())


def test_rne_matches_torch_on_float32_values():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(20000) * 10.0 ** rng.integers(-20, 20, 20000)).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(gemm.f64_to_bf16_rne_bits(x.astype(np.float64)), ref)


def test_rne_ties_and_single_rounding():
    # 1 + 2**-8 is halfway between 1 and 1 + 2**-7: ties to even -> 1.0 (0x3F80)
    # 1 + 3 * 2**-8 is halfway between 1 + 2**-7 and 1 + 2**-6: -> 1 + 2**-6 (0x3F82)
    # 1 + 2**-8 + 2**-40 is above the tie -> 1 + 2**-7 (0x3F81); rounding through
    # float32 first would land exactly on the tie and give 1.0 instead.
    x = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 1 + 2.0 ** -8 + 2.0 ** -40, -0.0, 0.0, 7168.0])
    np.testing.assert_array_equal(gemm.f64_to_bf16_rne_bits(x),
                                  np.array([0x3F80, 0x3F82, 0x3F81, 0x8000, 0x0000, 0x45E0],
                                           dtype=np.uint16))


def test_gemm_matches_bruteforce_triple_loop():
    rng = np.random.default_rng(2)
    W, m, K, N = 3, 2, 5, 4
    shards = [rng.integers(0, 2**16, size=(m, K), dtype=np.uint16) & 0xBFFF for _ in range(W)]
    b = rng.integers(0, 2**16, size=(K, N), dtype=np.uint16) & 0xBFFF
    ref = gemm.ag_gemm_ref(shards, b)
    for w in range(W):
        for i in range(m):
            for n in range(N):
                acc = 0.0
                for k in range(K):
                    a_val = float(gemm.bf16_bits_to_f64(shards[w][i:i + 1, k])[0])
                    b_val = float(gemm.bf16_bits_to_f64(b[k:k + 1, n])[0])
                    acc += a_val * b_val
                assert abs(ref[w * m + i, n] - acc) <= 1e-12 * max(1.0, abs(acc))


def test_gemm_integer_inputs_exact():
    rng = np.random.default_rng(3)
    W, m, K, N = 4, 3, 64, 5
    ai = [rng.integers(-1, 2, size=(m, K)) for _ in range(W)]
    bi = rng.integers(-1, 2, size=(K, N))
    to_bits = lambda a: gemm.f64_to_bf16_rne_bits(a.astype(np.float64))
    ref = gemm.ag_gemm_ref([to_bits(a) for a in ai], to_bits(bi))
    np.testing.assert_array_equal(ref, (np.concatenate(ai) @ bi).astype(np.float64))


def test_rows_ref_matches_full():
    rng = np.random.default_rng(4)
    shards = [rng.integers(0, 2**16, size=(4, 6), dtype=np.uint16) & 0xBFFF for _ in range(3)]
    b = rng.integers(0, 2**16, size=(6, 5), dtype=np.uint16) & 0xBFFF
    full = gemm.ag_gemm_ref(shards, b)
    rows = np.array([0, 5, 11, 7])
    np.testing.assert_array_equal(gemm.ag_gemm_rows_ref(shards, b, rows), full[rows])


def test_rel_error_definition():
    ref = np.array([1.0, -2.0, 0.0, 4.0])
    tau = 0.01 * np.sqrt((1 + 4 + 0 + 16) / 4)
    c = ref + np.array([0.01, 0.0, 0.001, 0.0])
    assert abs(gemm.rel_error(c, ref) - max(0.01, 0.001 / tau)) < 1e-15
    assert gemm.rel_error(ref, ref) == 0.0
    assert abs(gemm.normwise_error(c, ref) - 0.01 / 4.0) < 1e-15


def test_allgather_rows_is_oracle_allgather():
    shards = [np.arange(12, dtype=np.uint16).reshape(3, 4) + 100 * w for w in range(4)]
    np.testing.assert_array_equal(gemm.allgather_rows(shards), oracle.allgather(shards))


# ---- GEMM + ReduceScatter --------------------------------------------------------

def _bf16_ints(rng, shape, lo=-2, hi=3):
    """Small integers as bf16 bit patterns (exact in bf16)."""
    v = rng.integers(lo, hi, size=shape).astype(np.float64)
    return gemm.f64_to_bf16_rne_bits(v)


def test_gemm_rs_matches_bruteforce_loops():
    """out_j[i, n] = sum_r sum_k x1_r[j*m/W + i, k] * x2_r[k, n], written out as loops."""
    rng = np.random.default_rng(3)
    W, m, K, N = 3, 6, 4, 5
    a = [_bf16_ints(rng, (m, K)) for _ in range(W)]
    bt = [_bf16_ints(rng, (N, K)) for _ in range(W)]
    got = gemm.gemm_rs_ref(a, bt)
    mj = m // W
    for j in range(W):
        for i in range(mj):
            for n in range(N):
                want = 0.0
                for r in range(W):
                    for k in range(K):
                        want += (gemm.bf16_bits_to_f64(a[r][j * mj + i, k]) *
                                 gemm.bf16_bits_to_f64(bt[r][n, k]))
                assert got[j][i, n] == want


def test_gemm_rs_w1_is_plain_matmul():
    rng = np.random.default_rng(4)
    a = _bf16_ints(rng, (7, 9))
    bt = _bf16_ints(rng, (5, 9))
    got = gemm.gemm_rs_ref([a], [bt])[0]
    want = gemm.bf16_bits_to_f64(a) @ gemm.bf16_bits_to_f64(bt).T
    np.testing.assert_array_equal(got, want)


def test_gemm_rs_scatter_and_reduce_are_independent_of_each_other():
    """Concatenating the scattered blocks gives the sum of the per-rank products;
    scaling one rank's x2 scales only that rank's contribution."""
    rng = np.random.default_rng(5)
    W, m, K, N = 4, 8, 6, 3
    a = [_bf16_ints(rng, (m, K)) for _ in range(W)]
    bt = [_bf16_ints(rng, (N, K)) for _ in range(W)]
    full = np.concatenate(gemm.gemm_rs_ref(a, bt), axis=0)
    parts = [gemm.bf16_bits_to_f64(x) @ gemm.bf16_bits_to_f64(y).T for x, y in zip(a, bt)]
    np.testing.assert_array_equal(full, sum(parts))
    bt2 = list(bt)
    bt2[1] = gemm.f64_to_bf16_rne_bits(2.0 * gemm.bf16_bits_to_f64(bt[1]))
    full2 = np.concatenate(gemm.gemm_rs_ref(a, bt2), axis=0)
    np.testing.assert_array_equal(full2 - full, parts[1])


def test_gemm_rs_rows_ref_matches_full():
    rng = np.random.default_rng(6)
    W, m, K, N = 4, 12, 5, 7
    a = [_bf16_ints(rng, (m, K)) for _ in range(W)]
    bt = [_bf16_ints(rng, (N, K)) for _ in range(W)]
    full = gemm.gemm_rs_ref(a, bt)
    for j in range(W):
        rows = np.array([0, 2, m // W - 1])
        np.testing.assert_array_equal(gemm.gemm_rs_rows_ref(a, bt, j, rows), full[j][rows])


def test_gemm_rs_rejects_uneven_rows():
    import pytest
    rng = np.random.default_rng(7)
    with pytest.raises(ValueError):
        gemm.gemm_rs_ref([_bf16_ints(rng, (5, 2))] * 2, [_bf16_ints(rng, (3, 2))] * 2)


def test_gemm_rs_planted_mistakes_are_caught():
    """Plausible slips in a ReduceScatter (wrong row block, missing rank, rows of the
    destination's own input, transposed operand) all disagree with the loop pin."""
    rng = np.random.default_rng(8)
    W, m, K, N = 3, 6, 4, 5
    a = [_bf16_ints(rng, (m, K)) for _ in range(W)]
    bt = [_bf16_ints(rng, (N, K)) for _ in range(W)]
    ok = gemm.gemm_rs_ref(a, bt)
    f = gemm.bf16_bits_to_f64
    mj = m // W
    mutants = {
        "row block of the next rank": [sum(f(x) @ f(y).T for x, y in zip(a, bt))[((j + 1) % W) * mj:((j + 1) % W + 1) * mj] for j in range(W)],
        "a rank left out": [sum(f(x) @ f(y).T for x, y in list(zip(a, bt))[1:])[j * mj:(j + 1) * mj] for j in range(W)],
        "only the destination's own partial": [(f(a[j]) @ f(bt[j]).T)[j * mj:(j + 1) * mj] for j in range(W)],
        "x2 not transposed": [sum(f(x)[:, :N] @ f(y)[:, :N] for x, y in zip(a, bt))[j * mj:(j + 1) * mj] if K >= N else None for j in range(W)],
    }
    for name, outs in mutants.items():
        differs = any(o is None or o.shape != ok[j].shape or not np.array_equal(o, ok[j])
                      for j, o in enumerate(outs))
        assert differs, f"mutant '{name}' agrees with the oracle"


def _one_hot_rows(count, K):
    """A 1 x K row of `count` ones then zeros, as bf16 bits."""
    v = np.zeros((1, K))
    v[0, :count] = 1.0
    return gemm.f64_to_bf16_rne_bits(v)


def test_gemm_rs_rounded_partials_hand_worked():
    """W=2, m=2, N=1, K=264, x2 all ones.  Rank 0's partial for row 0 is 257, which
    lies halfway between the bf16 neighbours 256 and 258 (spacing 2 on [256, 512))
    and rounds to the even significand, 256; rank 1's partial is 1.  Rounded
    partials: 256 + 1 = 257, stored as bf16 256 (0x4380).  Exact partials: 258,
    a bf16 value (0x4381)."""
    K = 264
    ones = gemm.f64_to_bf16_rne_bits(np.ones((1, K)))
    a = [np.concatenate([_one_hot_rows(257, K), _one_hot_rows(0, K)]),
         np.concatenate([_one_hot_rows(1, K), _one_hot_rows(0, K)])]
    bt = [ones, ones]
    exact = gemm.gemm_rs_ref(a, bt)
    rounded = gemm.gemm_rs_ref(a, bt, round_partials=True)
    assert exact[0][0, 0] == 258.0 and rounded[0][0, 0] == 257.0
    assert exact[1][0, 0] == 0.0 and rounded[1][0, 0] == 0.0
    assert int(gemm.f64_to_bf16_rne_bits(rounded[0])[0, 0]) == 0x4380
    assert int(gemm.f64_to_bf16_rne_bits(exact[0])[0, 0]) == 0x4381
    np.testing.assert_array_equal(gemm.gemm_rs_rows_ref(a, bt, 0, np.array([0]), round_partials=True),
                                  rounded[0])


def test_gemm_rs_rounded_partials_equal_exact_when_partials_are_bf16_values():
    """Integer partials of magnitude <= 256 are bf16 values: rounding changes nothing."""
    rng = np.random.default_rng(9)
    W, m, K, N = 4, 8, 64, 6  # |partial| <= 2 * 2 * 64 = 256
    a = [_bf16_ints(rng, (m, K)) for _ in range(W)]
    bt = [_bf16_ints(rng, (N, K)) for _ in range(W)]
    for x, y in zip(gemm.gemm_rs_ref(a, bt), gemm.gemm_rs_ref(a, bt, round_partials=True)):
        np.testing.assert_array_equal(x, y)


def test_gemm_rs_rounded_partials_match_torch_bf16_matmul():
    """Each rounded partial equals torch's float64 product cast to bf16 (a library
    conversion), summed over ranks."""
    rng = np.random.default_rng(10)
    W, m, K, N = 2, 4, 40, 5
    a = [gemm.f64_to_bf16_rne_bits(rng.standard_normal((m, K))) for _ in range(W)]
    bt = [gemm.f64_to_bf16_rne_bits(rng.standard_normal((N, K))) for _ in range(W)]
    tot = 0
    for x, y in zip(a, bt):
        p = torch.from_numpy(gemm.bf16_bits_to_f64(x)) @ torch.from_numpy(gemm.bf16_bits_to_f64(y)).T
        tot = tot + p.to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    got = np.concatenate(gemm.gemm_rs_ref(a, bt, round_partials=True))
    # the float64 -> float32 -> bf16 double rounding can differ from one rounding
    # only on the rare values within 2**-24 relative of a bf16 midpoint
    assert np.mean(got == tot) > 0.99
    np.testing.assert_allclose(got, tot, rtol=2 ** -7)
