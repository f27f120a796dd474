"""fp64 oracles of the AllGather+GEMM and GEMM+ReduceScatter workloads -- TEST
INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg use
this module; the GPU path never imports it.

Followed passages: the HyperParallel RFC, section 十 ("fused_all_gather_matmul"),
and "Triton-distributed Semantics", section "AllGather + GEMM Overlapping": W
row shards A_w (m_local x K) are gathered into G (W*m_local x K) with shard w at
rows [w*m_local, (w+1)*m_local); the consumer computes C = G @ B.

Reading taken: the RFC's formula line also names a ReduceScatter, but its
example returns an (m_total, n) product, which only C = G @ B has; the oracle
computes C = G @ B with no reduction across ranks.

GEMM + ReduceScatter (the RFC, section 十, "fused_matmul_reduce_scatter"; and
"Triton-distributed Semantics", section "GEMM + ReduceScatter Overlapping"):
output = ReduceScatter(x1 @ x2).  Rank r holds x1_r (m x K) and x2_r (K x N);
its product is an (m x N) partial; the ReduceScatter sums the W partials and
gives rank j rows [j*m/W, (j+1)*m/W) of the sum (reading: an even row split, m
divisible by W).  The pages do not fix the partials' type.  Reading taken: the
partials are exact (the GPU keeps them in fp32); as an option, each partial is
the bf16 tensor a framework's matmul of bf16 operands returns, rounded before
the ReduceScatter adds them (``round_partials=True`` here).

bf16 inputs convert exactly to float64 (every bf16 value is a float64 value),
so ``ref`` is the exact product up to float64 summation rounding.
"""
from __future__ import annotations

from typing import List

import numpy as np


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly: bf16 is the top half of a float32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f64_to_bf16_rne_bits(x: np.ndarray) -> np.ndarray:
    """float64 -> bf16 bit patterns, round to nearest with ties to even, in one rounding.

    bf16 carries 8 significant bits.  With x = m * 2**k and 0.5 <= |m| < 1
    (``frexp``), the nearest bf16 value is round_half_even(m * 256) / 256 * 2**k;
    that value is exact in float32, whose top 16 bits are then the bf16 pattern.
    Zero maps to +/-0.  Values below bf16's normal range or beyond its largest
    finite value are rejected rather than guessed.
    """
    f = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(f)):
        raise ValueError("only finite values are supported")
    m, k = np.frexp(f)
    q = np.round(m * 256.0)  # numpy rounds halves to even
    v = np.ldexp(q / 256.0, k)
    nz = v != 0.0
    if np.any(np.abs(v[nz]) < 2.0 ** -126) or np.any(np.abs(v) > 3.3895313892515355e38):
        raise ValueError("value outside bf16's normal range")
    bits32 = v.astype(np.float32).view(np.uint32)
    if np.any(bits32 & np.uint32(0xFFFF)):
        raise AssertionError("rounded value is not a bf16 value")
    out = (bits32 >> np.uint32(16)).astype(np.uint16)
    # keep the sign of zero inputs
    zero_neg = (f == 0.0) & np.signbit(f)
    return np.where(zero_neg, np.uint16(0x8000), out).astype(np.uint16)


def allgather_rows(shards: List[np.ndarray]) -> np.ndarray:
    """G = shards stacked in rank order (shard w at rows [w*m, (w+1)*m))."""
    return np.concatenate([np.asarray(s) for s in shards], axis=0)


def ag_gemm_ref(shards_bits: List[np.ndarray], b_bits: np.ndarray) -> np.ndarray:
    """C = AllGather(A) @ B in float64 from bf16 bit patterns."""
    g = bf16_bits_to_f64(allgather_rows(shards_bits))
    b = bf16_bits_to_f64(b_bits)
    return g @ b


def ag_gemm_rows_ref(shards_bits: List[np.ndarray], b_bits: np.ndarray,
                     rows: np.ndarray) -> np.ndarray:
    """Selected rows of C (for sampled checks at full size)."""
    m_local = shards_bits[0].shape[0]
    a = np.stack([bf16_bits_to_f64(shards_bits[int(r) // m_local][int(r) % m_local])
                  for r in rows])
    return a @ bf16_bits_to_f64(b_bits)


def _partial(a: np.ndarray, bt: np.ndarray, round_partials: bool) -> np.ndarray:
    """x1_r @ x2_r in float64; with round_partials, as the bf16 tensor a framework's
    matmul of bf16 operands returns (the exact product rounded once to bf16,
    nearest even)."""
    p = bf16_bits_to_f64(a) @ bf16_bits_to_f64(bt).T
    return bf16_bits_to_f64(f64_to_bf16_rne_bits(p)) if round_partials else p


def gemm_rs_ref(a_bits: List[np.ndarray], bt_bits: List[np.ndarray],
                round_partials: bool = False) -> List[np.ndarray]:
    """out_j = (sum_r x1_r @ x2_r)[j*m/W : (j+1)*m/W] in float64.

    HyperParallel RFC, section 十, fused_matmul_reduce_scatter: output =
    ReduceScatter(x1 @ x2).  a_bits[r]: x1_r as bf16 bits (m x K); bt_bits[r]:
    x2_r transposed, bf16 bits (N x K), so x2_r = bt_bits[r].T.  The sum is taken
    in float64 either over the exact per-rank products or (round_partials) over
    the per-rank products rounded to bf16 first.
    """
    W = len(a_bits)
    m = a_bits[0].shape[0]
    if m % W:
        raise ValueError("m must be divisible by W")
    mj = m // W
    total = None
    for a, bt in zip(a_bits, bt_bits):
        part = _partial(a, bt, round_partials)
        total = part if total is None else total + part
    return [total[j * mj:(j + 1) * mj] for j in range(W)]


def gemm_rs_rows_ref(a_bits: List[np.ndarray], bt_bits: List[np.ndarray], j: int,
                     rows: np.ndarray, round_partials: bool = False) -> np.ndarray:
    """Selected rows of out_j (for sampled checks at full size)."""
    W = len(a_bits)
    mj = a_bits[0].shape[0] // W
    idx = j * mj + np.asarray(rows, dtype=np.int64)
    total = None
    for a, bt in zip(a_bits, bt_bits):
        part = _partial(a[idx], bt, round_partials)
        total = part if total is None else total + part
    return total


def rel_error(c: np.ndarray, ref: np.ndarray) -> float:
    """max_i |c_i - ref_i| / max(|ref_i|, tau), tau = 0.01 * RMS(ref).

    The floor tau keeps entries whose exact value is close to 0 from turning an
    absolute error at the level of bf16 output rounding into an unbounded ratio.
    """
    c = np.asarray(c, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    tau = 0.01 * float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    denom = np.maximum(np.abs(ref), tau)
    if denom.size == 0:
        return 0.0
    denom = np.where(denom == 0.0, 1.0, denom)
    return float(np.max(np.abs(c - ref) / denom))


def normwise_error(c: np.ndarray, ref: np.ndarray) -> float:
    """max |c - ref| / max |ref|."""
    c = np.asarray(c, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    m = float(np.max(np.abs(ref))) if ref.size else 0.0
    return float(np.max(np.abs(c - ref))) / (m if m else 1.0)
