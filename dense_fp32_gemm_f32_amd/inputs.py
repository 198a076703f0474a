"""Seeded synthetic inputs for the GEMM workloads.

This module only draws random numbers and lays them out in memory; it holds
none of the product's arithmetic, so both the HIP path and the CPU oracle can
be fed from it.

The pages time square random fp32 matrices (4096 x 4096 in "Optimizing a
WebGPU Matmul Kernel using Subgroups", 2048 x 2048 in "GPU compute shaders",
1024 x 1024 on the ybb.press page, N = 512 in "WebGPU 行列積の限界を測る") and
do not state the distribution.  The workloads below fix one per shape.

Recipe: a CPU ``torch.Generator`` seeded with the workload's seed draws A
first, then B, as dense logical matrices; each is then copied into a buffer
whose rows are ``ld`` elements apart.  Padding elements hold NaN so that a
kernel that reads or writes outside the logical window is caught.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch

PAD_FILL = float("nan")


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    dist_a: str
    dist_b: str
    seed: int        # float variant
    int_seed: int    # integer {-2..2} variant
    lda: int | None = None
    ldb: int | None = None
    ldc: int | None = None

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K

    @property
    def algo_bytes(self) -> int:
        """Compulsory HBM bytes: read A and B once, write C once (fp32)."""
        return 4 * (self.M * self.K + self.K * self.N + self.M * self.N)


_SKINNY_K = 8192
WORKLOADS = {
    "square_512": Workload("square_512", 512, 512, 512, "u11", "u11", 1001, 2001),
    "square_1024": Workload("square_1024", 1024, 1024, 1024, "u11", "u11", 1002, 2002),
    "square_4096": Workload("square_4096", 4096, 4096, 4096, "u11", "u11", 1003, 2003),
    "ragged_2047x3001x1531": Workload("ragged_2047x3001x1531", 2047, 3001, 1531,
                                      "normal", "normal", 1004, 2004,
                                      lda=1531, ldb=3001, ldc=3001),
    "skinny_8x8192x8192": Workload("skinny_8x8192x8192", 8, 8192, _SKINNY_K,
                                   "normal", "u_inv_sqrt_k", 1005, 2005),
}
HEADLINE = "square_4096"
SKINNY = "skinny_8x8192x8192"

# One GPU's share of a product split 8 ways (each share stored packed on its
# own GPU).  Along M or N a share is a whole product of its own; along K it
# is a full-size partial C that a reduce-scatter would add up.
SHARD_WAYS = 8
SHARDS = {
    "square_4096_split_m": Workload("square_4096_split_m", 512, 4096, 4096, "u11", "u11",
                                    1013, 2013),
    "square_4096_split_n": Workload("square_4096_split_n", 4096, 512, 4096, "u11", "u11",
                                    1023, 2023),
    "square_4096_split_k": Workload("square_4096_split_k", 4096, 4096, 512, "u11", "u11",
                                    1033, 2033),
    "skinny_8x8192x8192_split_n": Workload("skinny_8x8192x8192_split_n", 8, 1024, _SKINNY_K,
                                           "normal", "u_inv_sqrt_k", 1015, 2015),
}
SHARD_OF = {"square_4096_split_m": HEADLINE, "square_4096_split_n": HEADLINE,
            "square_4096_split_k": HEADLINE, "skinny_8x8192x8192_split_n": SKINNY}


def _draw(dist: str, rows: int, cols: int, g: torch.Generator, K: int) -> torch.Tensor:
    if dist == "u11":
        return torch.empty(rows, cols).uniform_(-1.0, 1.0, generator=g)
    if dist == "normal":
        return torch.randn(rows, cols, generator=g)
    if dist == "u_inv_sqrt_k":
        s = 1.0 / math.sqrt(K)
        return torch.empty(rows, cols).uniform_(-s, s, generator=g)
    if dist == "int2":
        return torch.randint(-2, 3, (rows, cols), generator=g).float()
    raise ValueError(f"unknown distribution {dist!r}")


def embed(x: torch.Tensor, ld: int, fill: float = PAD_FILL) -> torch.Tensor:
    """Return a (rows x ld) buffer holding ``x`` in its first columns; the
    result's ``[:, :cols]`` view is what a caller passes with pitch ``ld``."""
    rows, cols = x.shape
    if ld < cols:
        raise ValueError(f"ld {ld} < row length {cols}")
    if ld == cols:
        return x.contiguous()
    buf = torch.full((rows, ld), fill, dtype=x.dtype)
    buf[:, :cols] = x
    return buf


def make_ab(M: int, N: int, K: int, dist_a: str, dist_b: str, seed: int,
            lda: int | None = None, ldb: int | None = None):
    """Draw A (M x K) then B (K x N) on the CPU.  Returns row-pitched views
    ``(A, B)``: ``A.stride(0) == lda`` and ``B.stride(0) == ldb``."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    A = _draw(dist_a, M, K, g, K)
    B = _draw(dist_b, K, N, g, K)
    lda = K if lda is None else lda
    ldb = N if ldb is None else ldb
    Ab = embed(A, max(lda, 1))
    Bb = embed(B, max(ldb, 1))
    return Ab[:, :K], Bb[:, :N]


def workload_inputs(w: Workload | str, integer: bool = False):
    """A and B of a named workload, float or integer {-2..2} variant."""
    if isinstance(w, str):
        w = WORKLOADS[w] if w in WORKLOADS else SHARDS[w]
    if integer:
        return make_ab(w.M, w.N, w.K, "int2", "int2", w.int_seed, w.lda, w.ldb)
    return make_ab(w.M, w.N, w.K, w.dist_a, w.dist_b, w.seed, w.lda, w.ldb)


def int_matrix(rows: int, cols: int, seed: int, lo: int = -2, hi: int = 2) -> torch.Tensor:
    g = torch.Generator(device="cpu").manual_seed(seed)
    return torch.randint(lo, hi + 1, (rows, cols), generator=g).float()


def uniform_matrix(rows: int, cols: int, seed: int, lo: float = -1.0, hi: float = 1.0) -> torch.Tensor:
    g = torch.Generator(device="cpu").manual_seed(seed)
    return torch.empty(rows, cols).uniform_(lo, hi, generator=g)


def draw_matrix(rows: int, cols: int, dist: str, seed: int) -> torch.Tensor:
    """One rows x cols matrix of the named distribution from its own seed
    (``u_inv_sqrt_k`` scales by the row length ``cols``)."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    return _draw(dist, rows, cols, g, cols)
