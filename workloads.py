"""Seeded synthetic inputs for single-precision GEMM, C = A.B (row-major FP32).

This module only draws random matrices; it holds no matrix-multiply arithmetic.
Both the CPU oracle (``oracle/``) and the HIP library's tests and benchmark draw
their inputs from here, so the two sides see identical bytes.

Shapes follow the pages' workloads: square N x N problems (ratcatcher.ru
"Matrix multiplication: naive and tiled", section 1, N = 1024; GPU Parallel Book
ch. 9, section 9.1, N = 4096) and a general M, N, K problem (CUDA Handbook
section 17.3, the ``sgemm_cache(M, N, K, ...)`` signature).

Random-number convention (the pages do not fix one):
  * ``torch.Generator().manual_seed(seed)`` on the CPU;
  * A (M x K) is drawn first, then B (K x N), from the same generator;
  * "uniform" = 2*rand - 1, which is exact in FP32 (values are multiples of
    2**-23 in [-1, 1)); "normal" = randn;
  * the integer variant draws ``randint(-4, 5)`` from a fresh generator with the
    same seed and casts to FP32.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    lda: int
    ldb: int
    ldc: int
    dist: str  # "uniform" | "normal"
    seed: int

    @property
    def flops(self) -> int:
        """2*M*N*K: one multiply and one add per (i, j, k) term (GPU Parallel
        Book ch. 9, section 9.1; ratcatcher.ru page, section 1)."""
        return 2 * self.M * self.N * self.K

    @property
    def min_bytes(self) -> int:
        """Compulsory traffic: read A and B once, write C once, 4 bytes each
        (GPU Parallel Book ch. 9, section 9.1, minimum traffic 3N^2 elements)."""
        return 4 * (self.M * self.K + self.K * self.N + self.M * self.N)


WORKLOADS = [
    Workload("square256", 256, 256, 256, 256, 256, 256, "uniform", 0),
    Workload("square1024", 1024, 1024, 1024, 1024, 1024, 1024, "uniform", 1),
    Workload("square4096", 4096, 4096, 4096, 4096, 4096, 4096, "normal", 2),
    Workload("ragged3001x2047x1537", 3001, 2047, 1537, 1537, 2047, 2047, "uniform", 3),
    Workload("square8192", 8192, 8192, 8192, 8192, 8192, 8192, "uniform", 4),
]

BY_NAME = {w.name: w for w in WORKLOADS}


def draw(M: int, N: int, K: int, seed: int, dist: str = "uniform"):
    """Return (A, B) as contiguous FP32 CPU tensors, A is M x K, B is K x N."""
    g = torch.Generator().manual_seed(seed)
    if dist == "uniform":
        A = 2.0 * torch.rand((M, K), generator=g, dtype=torch.float32) - 1.0
        B = 2.0 * torch.rand((K, N), generator=g, dtype=torch.float32) - 1.0
    elif dist == "normal":
        A = torch.randn((M, K), generator=g, dtype=torch.float32)
        B = torch.randn((K, N), generator=g, dtype=torch.float32)
    elif dist == "int4":
        A = torch.randint(-4, 5, (M, K), generator=g).to(torch.float32)
        B = torch.randint(-4, 5, (K, N), generator=g).to(torch.float32)
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    return A.contiguous(), B.contiguous()


def inputs(w: Workload, integer: bool = False):
    """Inputs of a named workload; ``integer=True`` gives the {-4..4} variant."""
    return draw(w.M, w.N, w.K, w.seed, "int4" if integer else w.dist)


def embed(X: torch.Tensor, ld: int, fill: float = float("nan")) -> torch.Tensor:
    """Place the rows of X in a buffer of row stride ``ld`` >= X.shape[1].

    Returns a (rows x ld) tensor whose first X.shape[1] columns are X and whose
    padding columns hold ``fill`` (NaN by default, so any read of the padding
    poisons a result).
    """
    rows, cols = X.shape
    if ld < cols:
        raise ValueError("ld smaller than the row length")
    buf = torch.full((rows, ld), fill, dtype=torch.float32)
    buf[:, :cols] = X
    return buf


def as_numpy(X: torch.Tensor) -> np.ndarray:
    return np.ascontiguousarray(X.numpy())
