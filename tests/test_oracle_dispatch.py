"""Pins of the dispatch oracle (forward All2All, the combine's inverse).

"Reverse All2All (EP MoE Distributed Kernel)", sections "Reverse All2All
Operator Semantics" and "EP MoE Scenario": out_r[j*S+s, h, d] = in_j[s, r*H+h, d].
Pinned by a closed form on iota inputs, a numpy transpose, round trips through
the independently pinned combine oracle in both orders, and planted mistakes in
a copy of the C code that the closed form must catch.
"""
import ctypes
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

import oracle

SHAPES = [(2, 8, 4, 16), (3, 7, 1, 12), (1, 5, 3, 4), (4, 3, 5, 2), (5, 1, 2, 3)]


def iota_dispatch_inputs(W, S, H, D):
    """in_j[s, c, d] = j*S*H*W*D + (s*H*W + c)*D + d (each rank's own global iota)."""
    n = S * H * W * D
    return [(np.arange(n, dtype=np.int64) + j * n).reshape(S, H * W, D) for j in range(W)]


def closed_form(r, W, S, H, D):
    """out_r[j*S+s, h, d] written out from the definition, value by value."""
    out = np.empty((S * W, H, D), dtype=np.int64)
    n = S * H * W * D
    for j in range(W):
        for s in range(S):
            for h in range(H):
                for d in range(D):
                    out[j * S + s, h, d] = j * n + (s * H * W + r * H + h) * D + d
    return out


@pytest.mark.parametrize("W,S,H,D", SHAPES)
def test_iota_closed_form(W, S, H, D):
    ins = iota_dispatch_inputs(W, S, H, D)
    for r, got in enumerate(oracle.dispatch(ins)):
        np.testing.assert_array_equal(got, closed_form(r, W, S, H, D))


@pytest.mark.parametrize("W,S,H,D", SHAPES)
def test_numpy_transpose(W, S, H, D):
    """Stack the inputs as [j][s][r][h][d]; out_r is the [r][j][s][h][d] view."""
    rng = np.random.default_rng(W * 31 + S)
    ins = [rng.integers(0, 2**31, size=(S, H * W, D), dtype=np.int64) for _ in range(W)]
    x = np.stack(ins).reshape(W, S, W, H, D)
    want = x.transpose(2, 0, 1, 3, 4).reshape(W, S * W, H, D)
    for r, got in enumerate(oracle.dispatch(ins)):
        np.testing.assert_array_equal(got, want[r])


@pytest.mark.parametrize("W,S,H,D", SHAPES)
@pytest.mark.parametrize("dtype", [np.uint8, np.uint16, np.float32, np.float64])
def test_round_trips_through_the_combine(W, S, H, D, dtype):
    """combine(dispatch(y)) == y and dispatch(combine(x)) == x, byte for byte."""
    rng = np.random.default_rng(7 * W + H)
    y = [rng.integers(0, 255, size=(S, H * W, D)).astype(dtype) for _ in range(W)]
    back = oracle.combine(oracle.dispatch(y))
    for a, b in zip(back, y):
        assert a.tobytes() == b.tobytes()
    x = [rng.integers(0, 255, size=(S * W, H, D)).astype(dtype) for _ in range(W)]
    back = oracle.dispatch(oracle.combine(x))
    for a, b in zip(back, x):
        assert a.tobytes() == b.tobytes()


def test_w1_is_identity_copy():
    y = [np.arange(5 * 3 * 4, dtype=np.int32).reshape(5, 3, 4)]
    np.testing.assert_array_equal(oracle.dispatch(y)[0], y[0])


MUTANTS = {
    "rows from the wrong rank block": ("o = ((j * S + s) * H + h) * D + d;",
                                       "o = ((s * W + j) * H + h) * D + d;"),
    "columns of the wrong rank": ("i = (s * (H * W) + r * H + h) * D + d;",
                                  "i = (s * (H * W) + j * H + h) * D + d;"),
    "dropped rank term": ("i = (s * (H * W) + r * H + h) * D + d;",
                          "i = (s * (H * W) + h) * D + d;"),
    "wrong input row stride": ("i = (s * (H * W) + r * H + h) * D + d;",
                               "i = (s * H + r * H + h) * D + d;"),
    "source from the destination's input": ("((const uint16_t *)in[j])[i]; break;\n                    case 4: ((uint32_t *)out_r)[o] = ((const uint32_t *)in[j])[i]; break;\n                    case 8: ((uint64_t *)out_r)[o] = ((const uint64_t *)in[j])[i];",
                                            "((const uint16_t *)in[r])[i]; break;\n                    case 4: ((uint32_t *)out_r)[o] = ((const uint32_t *)in[r])[i]; break;\n                    case 8: ((uint64_t *)out_r)[o] = ((const uint64_t *)in[r])[i];"),
}


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_planted_mistakes_are_caught():
    src = open(os.path.join(os.path.dirname(oracle.__file__), "combine.c")).read()
    with tempfile.TemporaryDirectory() as td:
        for name, (a, b) in MUTANTS.items():
            assert a in src, f"mutation site for '{name}' not found"
            c = os.path.join(td, "m.c")
            so = os.path.join(td, name.replace(" ", "_").replace("'", "") + ".so")
            with open(c, "w") as f:
                f.write(src.replace(a, b, 1))
            subprocess.run(["gcc", "-O1", "-shared", "-fPIC", c, "-o", so], check=True,
                           capture_output=True)
            lib = ctypes.CDLL(so)
            i64 = ctypes.c_int64
            lib.oracle_dispatch_dest.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p,
                                                 i64, i64, i64, i64, i64, i64]
            caught = False
            for (W, S, H, D) in [(2, 8, 4, 16), (3, 7, 1, 12), (2, 2, 7, 9)]:
                ins = iota_dispatch_inputs(W, S, H, D)
                ptrs = (ctypes.c_void_p * W)(*[x.ctypes.data for x in ins])
                for r in range(W):
                    buf = np.zeros(S * H * W * D * 64, dtype=np.int64)  # a mutant may overrun
                    lib.oracle_dispatch_dest(ptrs, buf.ctypes.data, r, W, S, H, D, 8)
                    got = buf[:S * H * W * D].reshape(S * W, H, D)
                    if not np.array_equal(got, closed_form(r, W, S, H, D)):
                        caught = True
            assert caught, f"planted mistake '{name}' was not caught by the closed-form pin"
