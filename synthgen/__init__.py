"""Seeded synthetic inputs for the Reverse All2All combine, the AllGather+GEMM and
GEMM+ReduceScatter workloads and the variable-size AllToAll.

This module holds the workload definitions (shapes, element types, value
distributions, seeds and tiling) and the generators that turn them into host
arrays.  It holds none of the combine's or the GEMM's arithmetic: the CPU
oracle (``oracle/``) and the GPU path (``moe_all2all_combine_amd``) both consume
what it returns, and it imports neither of them.

Recipe (one reading, fixed so every run is reproducible):

* a torch CPU ``Generator().manual_seed(seed)`` per workload;
* values are drawn in float32 one simulated rank at a time, rank 0 first, from
  that one generator (``uniform_(-1, 1)`` or ``randn() * std``);
* bf16 workloads round the float32 sample to bf16 with torch's
  round-to-nearest-even conversion;
* the bytes are returned as numpy arrays of the same width (uint16 for bf16, so
  nothing downstream ever interprets them as floats unless it means to).

The shapes, tiles and distributions follow the workloads the Reverse All2All
page ("Reverse All2All (EP MoE Distributed Kernel)", section "Reverse All2All
Operator Semantics") and the HyperParallel RFC (section 十, fused_all_gather_matmul)
describe: per simulated rank an expert-output tensor of shape (S*W, H, D).
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np
import torch

# element type name -> (bytes per element, numpy dtype used to carry the bytes)
ELEM = {
    "u8": (1, np.uint8),
    "bf16": (2, np.uint16),
    "f16": (2, np.uint16),
    "i32": (4, np.int32),
    "f32": (4, np.float32),
    "f64": (8, np.float64),
    "i64": (8, np.int64),
}

PROTOCOL_SET = "set"
PROTOCOL_ADD = "add"


@dataclasses.dataclass(frozen=True)
class CombineWorkload:
    """One Reverse All2All workload: W simulated ranks, each with an (S*W, H, D) input."""

    name: str
    W: int
    S: int
    H: int
    D: int
    dtype: str            # key of ELEM
    dist: str             # "iota" | "uniform" | "normal" | "bytes"
    seed: int
    tile_s: int           # tokens per tile
    tile_h: int           # heads per tile
    tile_d: int           # elements of D per tile
    protocol: str         # PROTOCOL_SET | PROTOCOL_ADD
    std: float = 1.0
    straggler: bool = False

    @property
    def elem_bytes(self) -> int:
        return ELEM[self.dtype][0]

    @property
    def np_dtype(self):
        return ELEM[self.dtype][1]

    @property
    def rows(self) -> int:
        return self.S * self.W

    @property
    def bytes_per_rank(self) -> int:
        return self.S * self.W * self.H * self.D * self.elem_bytes

    @property
    def algorithmic_bytes(self) -> int:
        """Every input element read once plus every output element written once."""
        return 2 * self.W * self.bytes_per_rank


@dataclasses.dataclass(frozen=True)
class AgGemmWorkload:
    """AllGather of W row shards of A followed by C = gather(A) @ B."""

    name: str
    W: int
    m_local: int
    K: int
    N: int
    tile_rows: int
    seed_a: int
    seed_b: int
    std: float


WORKLOADS = {
    # correctness case: W=2, int32 values equal to the global iota
    "iota_w2_s8_h4_d16_i32": CombineWorkload(
        "iota_w2_s8_h4_d16_i32", W=2, S=8, H=4, D=16, dtype="i32", dist="iota", seed=0,
        tile_s=8, tile_h=4, tile_d=16, protocol=PROTOCOL_SET),
    # EP combine, 64-token x 1-head x 128 tiles, ADD-to-W tile signals
    "ep_combine_w8_s512_h16_d128_bf16": CombineWorkload(
        "ep_combine_w8_s512_h16_d128_bf16", W=8, S=512, H=16, D=128, dtype="bf16",
        dist="uniform", seed=0, tile_s=64, tile_h=1, tile_d=128, protocol=PROTOCOL_ADD),
    # MoE-combine shaped, ~470 MB of input per simulated rank, 32 x 7168 tiles
    "moe_combine_w8_s4096_h1_d7168_bf16": CombineWorkload(
        "moe_combine_w8_s4096_h1_d7168_bf16", W=8, S=4096, H=1, D=7168, dtype="bf16",
        dist="normal", seed=1, tile_s=32, tile_h=1, tile_d=7168, protocol=PROTOCOL_ADD),
    # straggler: one source slice's producers delayed, SET per piece
    "straggler_w16_s2048_h32_d128_f32": CombineWorkload(
        "straggler_w16_s2048_h32_d128_f32", W=16, S=2048, H=32, D=128, dtype="f32",
        dist="uniform", seed=2, tile_s=64, tile_h=1, tile_d=128, protocol=PROTOCOL_SET,
        straggler=True),
}

AG_GEMM = AgGemmWorkload("ag_gemm_w8_m1024_k7168_n4096_bf16", W=8, m_local=1024, K=7168,
                         N=4096, tile_rows=128, seed_a=3, seed_b=4, std=0.02)


@dataclasses.dataclass(frozen=True)
class GemmRsWorkload:
    """GEMM + ReduceScatter: rank r holds x1_r (m x K) and x2_r (K x N, passed
    transposed); rank j receives rows [j*m/W, (j+1)*m/W) of sum_r x1_r @ x2_r."""

    name: str
    W: int
    m: int
    K: int
    N: int
    seed_a: int
    seed_b: int
    std: float


# The ReduceScatter counterpart of the AllGather+GEMM workload: the same 8192 x
# 4096 output and the same FLOPs, with K = 7168 split over the 8 ranks (each
# rank's x1_r is its K-slice of the activations, x2_r its K-slice of the weight).
GEMM_RS = GemmRsWorkload("gemm_rs_w8_m8192_k896_n4096_bf16", W=8, m=8192, K=896, N=4096,
                         seed_a=6, seed_b=7, std=0.02)


def small_workload(W: int, S: int, H: int, D: int, dtype: str = "bf16", seed: int = 0,
                   tile=(None, None, None), protocol: str = PROTOCOL_ADD,
                   dist: Optional[str] = None) -> CombineWorkload:
    """A reduced workload for tests (ragged shapes, edge cases)."""
    ts, th, td = tile
    if dist is None:
        dist = "uniform" if dtype in ("bf16", "f16", "f32", "f64") else "bytes"
    return CombineWorkload(
        f"w{W}_s{S}_h{H}_d{D}_{dtype}", W=W, S=S, H=H, D=D, dtype=dtype, dist=dist, seed=seed,
        tile_s=ts or min(S, 64), tile_h=th or 1, tile_d=td or D, protocol=protocol)


def _rank_values(wl: CombineWorkload, r: int, g: torch.Generator) -> np.ndarray:
    shape = (wl.S * wl.W, wl.H, wl.D)
    n = wl.S * wl.W * wl.H * wl.D
    if wl.dist == "iota":
        # value = r * (S*W*H*D) + flat index inside rank r's input
        base = r * n
        vals = np.arange(base, base + n, dtype=np.int64)
        return vals.astype(wl.np_dtype).reshape(shape)
    if wl.dist == "bytes":
        t = torch.randint(0, 256, (n * wl.elem_bytes,), dtype=torch.uint8, generator=g)
        return t.numpy().view(wl.np_dtype).reshape(shape)
    if wl.dist == "uniform":
        t = torch.empty(n, dtype=torch.float32).uniform_(-1.0, 1.0, generator=g)
    elif wl.dist == "normal":
        t = torch.randn(n, dtype=torch.float32, generator=g) * wl.std
    else:
        raise ValueError(wl.dist)
    if wl.dtype == "bf16":
        return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).reshape(shape)
    if wl.dtype == "f16":
        return t.to(torch.float16).view(torch.int16).numpy().view(np.uint16).reshape(shape)
    if wl.dtype == "f32":
        return t.numpy().reshape(shape)
    if wl.dtype == "f64":
        return t.to(torch.float64).numpy().reshape(shape)
    raise ValueError(wl.dtype)


def make_inputs(wl: CombineWorkload, ranks: Optional[List[int]] = None) -> List[np.ndarray]:
    """Per-rank input arrays of shape (S*W, H, D), drawn rank-major from one generator.

    ``ranks`` restricts the returned list to those ranks (the generator still
    advances through the earlier ranks so the values do not depend on it).
    """
    g = torch.Generator().manual_seed(wl.seed)
    want = set(range(wl.W)) if ranks is None else set(ranks)
    out = []
    for r in range(wl.W):
        v = _rank_values(wl, r, g)
        if r in want:
            out.append(v)
    return out


def straggler_rank(wl: CombineWorkload) -> int:
    """The delayed source slice: one draw from a generator seeded with the workload seed."""
    g = torch.Generator().manual_seed(wl.seed)
    return int(torch.randint(0, wl.W, (1,), generator=g).item())


def make_ag_gemm_inputs(wl: AgGemmWorkload = AG_GEMM, m_local: Optional[int] = None,
                        K: Optional[int] = None, N: Optional[int] = None, W: Optional[int] = None):
    """(list of W bf16 A shards as uint16 (m_local, K), bf16 B as uint16 (K, N))."""
    W = W or wl.W
    m_local = m_local or wl.m_local
    K = K or wl.K
    N = N or wl.N
    ga = torch.Generator().manual_seed(wl.seed_a)
    shards = []
    for _ in range(W):
        t = torch.randn(m_local * K, dtype=torch.float32, generator=ga) * wl.std
        shards.append(t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
                      .reshape(m_local, K))
    gb = torch.Generator().manual_seed(wl.seed_b)
    tb = torch.randn(K * N, dtype=torch.float32, generator=gb) * wl.std
    b = tb.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).reshape(K, N)
    return shards, b


def make_integer_ag_gemm_inputs(W: int, m_local: int, K: int, N: int, seed: int = 5):
    """bf16 A shards and B whose values are integers in {-1, 0, 1} (exactly representable)."""
    g = torch.Generator().manual_seed(seed)
    shards = []
    for _ in range(W):
        t = torch.randint(-1, 2, (m_local, K), generator=g).to(torch.float32)
        shards.append(t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
    tb = torch.randint(-1, 2, (K, N), generator=g).to(torch.float32)
    b = tb.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return shards, b


def make_gemm_rs_inputs(wl: GemmRsWorkload = GEMM_RS, m: Optional[int] = None,
                        K: Optional[int] = None, N: Optional[int] = None, W: Optional[int] = None,
                        integer: bool = False):
    """(list of W x1_r as bf16 bits (m, K), list of W x2_r^T as bf16 bits (N, K)).

    Normal(0, std) values, or (integer=True) integers in {-1, 0, 1}."""
    W = W or wl.W
    m = m or wl.m
    K = K or wl.K
    N = N or wl.N

    def draw(g, shape):
        if integer:
            t = torch.randint(-1, 2, shape, generator=g).to(torch.float32)
        else:
            t = torch.randn(shape, dtype=torch.float32, generator=g) * wl.std
        return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)

    ga = torch.Generator().manual_seed(wl.seed_a)
    gb = torch.Generator().manual_seed(wl.seed_b)
    a = [draw(ga, (m, K)) for _ in range(W)]
    bt = [draw(gb, (N, K)) for _ in range(W)]
    return a, bt


@dataclasses.dataclass(frozen=True)
class AllToAllvWorkload:
    """Variable-size AllToAll: rank r holds `rows` rows of `row_bytes` bytes and
    sends send_counts[r][j] of them to rank j, the counts of each rank a
    multinomial draw over the W destinations with Dirichlet(alpha) weights (the
    uneven token-to-expert routing of an MoE dispatch)."""

    name: str
    W: int
    rows: int
    row_bytes: int
    seed: int
    alpha: float


# MoE-shaped: 32768 rows of 7168 bf16 per rank (the same bytes per rank as the
# W=8, S=4096, H=1, D=7168 combine), routed unevenly.
ALLTOALLV = AllToAllvWorkload("alltoallv_w8_rows32768_row14336B", W=8, rows=32768,
                              row_bytes=7168 * 2, seed=12, alpha=4.0)


def make_alltoallv_counts(W: int, rows: int, seed: int, alpha: float = 4.0,
                          empty_pairs: int = 0) -> np.ndarray:
    """send_counts (W x W int64): row r sums to `rows`; `empty_pairs` (r, j) pairs,
    chosen by the same generator, are forced to 0 (their rows go to the next
    destination)."""
    rng = np.random.default_rng(seed)
    c = np.zeros((W, W), dtype=np.int64)
    for r in range(W):
        p = rng.dirichlet(np.full(W, alpha))
        c[r] = rng.multinomial(rows, p)
    for _ in range(empty_pairs):
        r, j = int(rng.integers(0, W)), int(rng.integers(0, W))
        c[r, (j + 1) % W] += c[r, j]
        c[r, j] = 0
    return c


def make_alltoallv_inputs(W: int, rows: int, row_bytes: int, seed: int) -> List[np.ndarray]:
    """W arrays of (rows, row_bytes) uniform random bytes, rank 0 first."""
    rng = np.random.default_rng(seed + 1000)
    return [np.frombuffer(rng.bytes(rows * row_bytes), dtype=np.uint8).reshape(rows, row_bytes).copy()
            for _ in range(W)]
