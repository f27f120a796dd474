"""Pins of the combine oracle against what the definition and mathematics fix.

None of these re-types the oracle's loop: they use a closed form on iota
inputs, hand-derived worked values, numpy's transpose, a brute-force scatter
written from the input side, and the permutation invariant.  A test at the
end plants mistakes in a copy of the oracle's C source and checks that the
pins catch each one.
"""
import itertools
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

import oracle
import synthgen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "iota_w2_s8_h4_d16_i32.txt")


def iota_inputs(W, S, H, D, dtype=np.int64):
    n = S * W * H * D
    return [np.arange(r * n, (r + 1) * n, dtype=np.int64).astype(dtype).reshape(S * W, H, D)
            for r in range(W)]


def closed_form(j, W, S, H, D):
    """out_j[s, c, d] for iota inputs: (c div H)*N + ((j*S + s)*H + c mod H)*D + d."""
    n = S * W * H * D
    s = np.arange(S)[:, None, None]
    c = np.arange(H * W)[None, :, None]
    d = np.arange(D)[None, None, :]
    return (c // H) * n + ((j * S + s) * H + c % H) * D + d


SHAPES = [(2, 8, 4, 16), (1, 3, 2, 5), (3, 7, 1, 12), (4, 5, 3, 1), (5, 1, 2, 3), (2, 2, 7, 9)]


@pytest.mark.parametrize("W,S,H,D", SHAPES)
def test_iota_closed_form(W, S, H, D):
    outs = oracle.combine(iota_inputs(W, S, H, D))
    for j in range(W):
        np.testing.assert_array_equal(outs[j], closed_form(j, W, S, H, D))


def test_worked_values_iota_w2():
    wl = synthgen.WORKLOADS["iota_w2_s8_h4_d16_i32"]
    outs = oracle.combine(synthgen.make_inputs(wl))
    rows = [l.split() for l in open(GOLDEN) if l.strip() and not l.startswith("#")]
    assert len(rows) >= 5
    for j, s, c, d, v in (map(int, r) for r in rows):
        assert outs[j][s, c, d] == v, (j, s, c, d)


@pytest.mark.parametrize("dtype", [np.uint8, np.uint16, np.uint32, np.uint64])
@pytest.mark.parametrize("W,S,H,D", [(3, 4, 2, 5), (2, 8, 4, 16), (4, 3, 1, 7)])
def test_numpy_transpose(dtype, W, S, H, D):
    rng = np.random.default_rng(W * 1000 + S * 100 + H * 10 + D)
    info = np.iinfo(dtype)
    ins = [rng.integers(0, info.max, size=(S * W, H, D), dtype=dtype, endpoint=True)
           for _ in range(W)]
    outs = oracle.combine(ins)
    # X[r, j, s, h, d] = in_r[j*S+s, h, d]; Y[j, s, r, h, d] = out_j[s, r*H+h, d]
    x = np.stack(ins).reshape(W, W, S, H, D)
    y = x.transpose(1, 2, 0, 3, 4).reshape(W, S, W * H, D)
    for j in range(W):
        np.testing.assert_array_equal(outs[j], y[j])


def test_bruteforce_scatter_all_tiny_shapes():
    """Scatter form, written from the input side: element (r, t, h, d) goes to
    rank t div S at row t mod S, column r*H + h."""
    count = 0
    for W, S, H, D in itertools.product(range(1, 4), range(1, 5), range(1, 4), range(1, 4)):
        rng = np.random.default_rng(count)
        ins = [rng.integers(0, 2**31, size=(S * W, H, D), dtype=np.int32) for _ in range(W)]
        expect = [np.full((S, H * W, D), -1, dtype=np.int32) for _ in range(W)]
        for r in range(W):
            for t in range(S * W):
                for h in range(H):
                    for d in range(D):
                        expect[t // S][t % S, r * H + h, d] = ins[r][t, h, d]
        outs = oracle.combine(ins)
        for j in range(W):
            np.testing.assert_array_equal(outs[j], expect[j], err_msg=str((W, S, H, D, j)))
        count += 1
    assert count == 3 * 4 * 3 * 3


@pytest.mark.parametrize("W,S,H,D", [(3, 5, 2, 3), (8, 4, 2, 8), (2, 1, 1, 1)])
def test_permutation_every_input_once(W, S, H, D):
    """Hit count: every input element appears exactly once across all outputs."""
    n = S * W * H * D
    outs = oracle.combine(iota_inputs(W, S, H, D, np.int64))
    allv = np.sort(np.concatenate([o.ravel() for o in outs]))
    np.testing.assert_array_equal(allv, np.arange(W * n))


def test_permutation_two_byte_elements():
    """For 2-byte elements: two passes, coding index mod 2**16 and index >> 16."""
    W, S, H, D = 4, 300, 3, 20  # W*n = 288000 > 2**16
    n = S * W * H * D
    idx = [np.arange(r * n, (r + 1) * n, dtype=np.int64).reshape(S * W, H, D) for r in range(W)]
    lo = oracle.combine([(a & 0xFFFF).astype(np.uint16) for a in idx])
    hi = oracle.combine([(a >> 16).astype(np.uint16) for a in idx])
    got = np.concatenate([(h.astype(np.int64) << 16 | l.astype(np.int64)).ravel()
                          for l, h in zip(lo, hi)])
    hits = np.bincount(got, minlength=W * n)
    assert hits.min() == 1 and hits.max() == 1


def test_source_of_matches_closed_form():
    W, S, H, D = 3, 5, 4, 6
    rng = np.random.default_rng(7)
    for _ in range(200):
        j, s, c, d = (int(rng.integers(W)), int(rng.integers(S)), int(rng.integers(H * W)),
                      int(rng.integers(D)))
        r, row, h = oracle.source_of(j, s, c, d, W, S, H, D)
        # value of in_r[row, h, d] under iota coding equals the closed form
        assert r * S * W * H * D + (row * H + h) * D + d == closed_form(j, W, S, H, D)[s, c, d]


def test_w1_is_identity_copy():
    ins = iota_inputs(1, 6, 2, 3)
    np.testing.assert_array_equal(oracle.combine(ins)[0], ins[0])


def test_allgather_stacks_rank_major():
    shards = [np.full((3, 4), w, dtype=np.uint16) for w in range(5)]
    g = oracle.allgather(shards)
    assert g.shape == (15, 4)
    for w in range(5):
        assert (g[3 * w:3 * w + 3] == w).all()


# ---- the pins have teeth: plant mistakes in a copy of the oracle -----------------

MUTANTS = {
    "source rows from the wrong rank": ("= IN_INDEX(j, s, h, d)", "= IN_INDEX(r, s, h, d)"),
    "transposed output columns": ("(r) * H + (h)", "(h) * W + (r)"),
    "dropped rank term": ("(r) * H + (h)", "(h)"),
    "wrong output row stride": ("((s) * (H * W))", "((s) * H)"),
    "wrong input row": ("(j) * S + (s)", "(s) * W + (j)"),
}


def _compile_mutant(src_text, tmpdir, name):
    c = os.path.join(tmpdir, name + ".c")
    so = os.path.join(tmpdir, name + ".so")
    with open(c, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", "-O1", "-shared", "-fPIC", c, "-o", so], check=True,
                   capture_output=True)
    return so


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_planted_mistakes_are_caught():
    import ctypes
    src = open(os.path.join(os.path.dirname(oracle.__file__), "combine.c")).read()
    with tempfile.TemporaryDirectory() as td:
        for name, (a, b) in MUTANTS.items():
            assert a in src, f"mutation site for '{name}' not found"
            so = _compile_mutant(src.replace(a, b, 1), td, name.replace(" ", "_"))
            lib = ctypes.CDLL(so)
            i64 = ctypes.c_int64
            lib.oracle_combine_dest.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p,
                                                i64, i64, i64, i64, i64, i64]
            caught = False
            for (W, S, H, D) in [(2, 8, 4, 16), (3, 7, 1, 12), (2, 2, 7, 9)]:
                ins = iota_inputs(W, S, H, D)
                ptrs = (ctypes.c_void_p * W)(*[x.ctypes.data for x in ins])
                for j in range(W):
                    # generous buffer: a mutant may index past the true output
                    buf = np.zeros((S * H * W * D) * 64, dtype=np.int64)
                    lib.oracle_combine_dest(ptrs, buf.ctypes.data, j, W, S, H, D, 8)
                    got = buf[:S * H * W * D].reshape(S, H * W, D)
                    if not np.array_equal(got, closed_form(j, W, S, H, D)):
                        caught = True
            assert caught, f"planted mistake '{name}' was not caught by the closed-form pin"


def test_combine_dest_rows_assembles_the_destination():
    """Row ranges of a destination computed separately (as a threaded caller would)
    assemble exactly the whole destination, for ranges of every size, including
    empty ones."""
    rng = np.random.default_rng(3)
    W, S, H, D = 3, 11, 2, 5
    ins = [rng.integers(0, 2**16, size=(S * W, H, D), dtype=np.uint16) for _ in range(W)]
    for j in range(W):
        want = oracle.combine_dest(ins, j)
        for cuts in ([0, S], [0, 4, 4, 9, S], [0, 1, 2, 3, 5, 8, S]):
            out = np.zeros((S, H * W, D), dtype=np.uint16)
            for a, b in zip(cuts[:-1], cuts[1:]):
                oracle.combine_dest_rows(ins, out, j, a, b)
            assert out.tobytes() == want.tobytes()
    with pytest.raises(ValueError):
        oracle.combine_dest_rows(ins, np.zeros((S, H * W, D), dtype=np.uint16), 0, 5, 3)
