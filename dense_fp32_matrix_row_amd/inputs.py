"""Seeded synthetic inputs for single-precision GEMM, shared by the tests, the
benchmark and the CPU reference checks.

This module holds no GEMM arithmetic: it only draws random matrices and lays
them out in row-major buffers with a leading dimension.  It is the one piece of
code that both the HIP path and the CPU reference are fed from.

The pages this library follows never state a value distribution for their
matrices (they time square FP32 problems at 1024, 2048, 4096 and 4097 on
otherwise unspecified data: "SGEMM 六级优化" K2 section 4096/4097 table;
"CUDA-Practice 04" performance tables).  The workloads here use i.i.d.
uniform[-1, 1] entries drawn in float64 and rounded to float32, A first, then
B, then C, from one PCG64 generator seeded per workload.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    """One square-or-not FP32 GEMM problem C <- alpha*A@B + beta*C."""

    name: str
    M: int
    N: int
    K: int
    alpha: float
    beta: float
    seed: int

    @property
    def flops(self) -> int:
        """Algorithmic floating-point operations, 2*M*N*K (one multiply and
        one add per term of every output's dot product)."""
        return 2 * self.M * self.N * self.K

    @property
    def algorithmic_bytes(self) -> int:
        """Algorithmic HBM bytes, 4*(M*K + K*N + 2*M*N): read A and B once,
        read and write C once."""
        return 4 * (self.M * self.K + self.K * self.N + 2 * self.M * self.N)


# The five problem sizes: 256^3, 1024^3 and 2048^3 with alpha=1, beta=0; the
# 4096^3 headline with alpha=0.5, beta=3 (exercises the beta*C read); and
# 4097^3 with alpha=beta=1, which breaks 16-byte row alignment and every
# power-of-two tile divisibility.  Seeds are 1000 + position.
WORKLOADS = (
    Workload("sgemm_256", 256, 256, 256, 1.0, 0.0, 1000),
    Workload("sgemm_1024", 1024, 1024, 1024, 1.0, 0.0, 1001),
    Workload("sgemm_2048", 2048, 2048, 2048, 1.0, 0.0, 1002),
    Workload("sgemm_4096", 4096, 4096, 4096, 0.5, 3.0, 1003),
    Workload("sgemm_4097", 4097, 4097, 4097, 1.0, 1.0, 1004),
)

WORKLOADS_BY_NAME = {w.name: w for w in WORKLOADS}


def uniform_f32(rng: np.random.Generator, shape, lo: float = -1.0, hi: float = 1.0) -> np.ndarray:
    """Draw float64 uniform[lo, hi) and round to float32 (round-to-nearest-even)."""
    return rng.uniform(lo, hi, size=shape).astype(np.float32)


def padded(mat: np.ndarray, ld: Optional[int], fill: float) -> np.ndarray:
    """Place a rows x cols matrix into a row-major buffer with row stride `ld`
    (>= cols).  Returns the flat buffer of length rows*ld (the last row's
    padding included, so guard values sit after every row).  The padding is
    set to `fill`."""
    rows, cols = mat.shape
    ld = cols if ld is None else ld
    if ld < cols:
        raise ValueError("leading dimension smaller than the row length")
    buf = np.full((rows, ld), fill, dtype=np.float32)
    buf[:, :cols] = mat
    return buf.reshape(-1)


def make_abc(M: int, N: int, K: int, seed: int):
    """Dense M x K, K x N and M x N float32 matrices, drawn A, then B, then C."""
    rng = np.random.default_rng(seed)
    A = uniform_f32(rng, (M, K))
    B = uniform_f32(rng, (K, N))
    C = uniform_f32(rng, (M, N))
    return A, B, C


def make_workload(w: Workload):
    """The dense inputs of a named workload."""
    return make_abc(w.M, w.N, w.K, w.seed)


def integer_abc(M: int, N: int, K: int, seed: int, lo: int = -8, hi: int = 8):
    """Matrices with integer entries in [lo, hi]: every partial dot product is
    an integer well below 2**24, so any summation order is exact in FP32."""
    rng = np.random.default_rng(seed)
    A = rng.integers(lo, hi + 1, size=(M, K)).astype(np.float32)
    B = rng.integers(lo, hi + 1, size=(K, N)).astype(np.float32)
    C = rng.integers(lo, hi + 1, size=(M, N)).astype(np.float32)
    return A, B, C


def permutation(n: int, seed: int) -> np.ndarray:
    """A random n x n permutation matrix as float32: row i has its single 1
    at column perm[i] (recover perm with argmax along rows)."""
    rng = np.random.default_rng(seed)
    perm = rng.permutation(n)
    P = np.zeros((n, n), dtype=np.float32)
    P[np.arange(n), perm] = 1.0
    return P
