"""Helpers of the GPU tests: lay out guarded device buffers, call the C ABI,
read results back and check that nothing outside the M x N window changed.

Buffers are row-major with a leading dimension; A's and B's row padding is
NaN (a read of it would poison results) and C's row padding, plus guard
regions before and after every buffer, hold a sentinel that must survive.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

from dense_fp32_matrix_row_amd import sgemm

SENTINEL = np.float32(-7.25e30)


@dataclasses.dataclass
class Case:
    M: int
    N: int
    K: int
    alpha: float
    beta: float
    A: np.ndarray  # M x K float32
    B: np.ndarray  # K x N float32
    C: np.ndarray  # M x N float32 (the C passed in)
    lda: Optional[int] = None
    ldb: Optional[int] = None
    ldc: Optional[int] = None
    a_off: int = 0   # elements between the allocation start and A (misalignment)
    b_off: int = 0
    c_off: int = 0


def _flat(mat: np.ndarray, ld: int, off: int, guard: int, fill_pad, fill_guard) -> np.ndarray:
    rows, cols = mat.shape
    body = np.full((rows, ld), fill_pad, dtype=np.float32)
    if rows and cols:
        body[:, :cols] = mat
    out = np.full(off + rows * ld + guard, fill_guard, dtype=np.float32)
    out[off:off + rows * ld] = body.reshape(-1)
    return out


def run(case: Case, level, stream=None, guard: int = 67):
    """Run one call; returns (C_out M x N float32, status).  Raises if a value
    outside the window of C changed.  `level` is a level number, None
    (hip_sgemm), or a callable taking hip_sgemm's twelve arguments."""
    M, N, K = case.M, case.N, case.K
    lda = max(1, K) if case.lda is None else case.lda
    ldb = max(1, N) if case.ldb is None else case.ldb
    ldc = max(1, N) if case.ldc is None else case.ldc
    hA = _flat(case.A, lda, case.a_off, guard, np.nan, np.nan)
    hB = _flat(case.B, ldb, case.b_off, guard, np.nan, np.nan)
    hC = _flat(case.C, ldc, case.c_off, guard, SENTINEL, SENTINEL)
    dA, dB, dC = (torch.from_numpy(x).cuda() for x in (hA, hB, hC))
    pa = dA.data_ptr() + 4 * case.a_off
    pb = dB.data_ptr() + 4 * case.b_off
    pc = dC.data_ptr() + 4 * case.c_off
    if level is None:
        st = sgemm.hip_sgemm(M, N, K, case.alpha, pa, lda, pb, ldb, case.beta, pc, ldc, stream)
    elif callable(level):
        st = level(M, N, K, case.alpha, pa, lda, pb, ldb, case.beta, pc, ldc, stream)
    else:
        st = sgemm.hip_sgemm_level(level, M, N, K, case.alpha, pa, lda, pb, ldb, case.beta, pc, ldc,
                                   stream)
    torch.cuda.synchronize()
    out = dC.cpu().numpy()
    # everything but the M x N window must be bit-identical to what was there
    window = np.zeros(out.shape, dtype=bool)
    if M and N:
        idx = case.c_off + (np.arange(M)[:, None] * ldc + np.arange(N)[None, :])
        window[idx.reshape(-1)] = True
    before = hC.view(np.uint32)
    after = out.view(np.uint32)
    changed = np.nonzero((before != after) & ~window)[0]
    if changed.size:
        raise AssertionError(f"{changed.size} elements outside the C window changed "
                             f"(first at flat index {changed[0]})")
    body = out[case.c_off:case.c_off + M * ldc].reshape(M, ldc)[:, :N] if M else np.zeros((0, N), np.float32)
    return body.copy(), st


class Resident:
    """Dense device copies of a large problem, reused across levels: A and B
    stay, C is restored from a pristine device copy before each call."""

    def __init__(self, A: np.ndarray, B: np.ndarray, C: np.ndarray):
        self.M, self.K = A.shape
        self.N = B.shape[1]
        self.dA = torch.from_numpy(A).cuda()
        self.dB = torch.from_numpy(B).cuda()
        self.dC0 = torch.from_numpy(C).cuda()
        self.dC = torch.empty_like(self.dC0)

    def call(self, level: Optional[int], alpha: float, beta: float, rows=None, stream=None):
        """Run on a fresh C; return C_out (all rows, or the selected ones) and status."""
        self.dC.copy_(self.dC0)
        args = (self.M, self.N, self.K, alpha, self.dA, self.K, self.dB, self.N, beta, self.dC,
                self.N, stream)
        st = sgemm.hip_sgemm(*args) if level is None else sgemm.hip_sgemm_level(level, *args)
        torch.cuda.synchronize()
        out = self.dC if rows is None else self.dC[torch.as_tensor(rows, device="cuda")]
        return out.cpu().numpy(), st
