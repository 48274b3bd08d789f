"""ctypes front end of the CPU reference (liboracle_sgemm.so) and the
normalised-error checker.

TEST INFRASTRUCTURE ONLY: only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import this module.  It never imports the HIP
library's package, and the HIP library never imports it.

The oracle computes ref = alpha * A @ B + beta * C in float64 with exact
float32 x float32 products summed in ascending k (see oracle_sgemm.c for the
passages it follows).  The checker implements the acceptance metric

    err = max_ij |C_gpu[i][j] - ref[i][j]| / den[i][j],
    den[i][j] = sum_k |A[i][k] * B[k][j]| + |beta * C[i][j]|,

where an element with den == 0 must come out exactly zero (either sign).  A
stricter variant scales the product part by |alpha| (den = |alpha| *
sum|a*b| + |beta*c|), which is the true scale of a float32 evaluation's
rounding error when |alpha| < 1.
"""

from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(HERE, "liboracle_sgemm.so")

_libs = {}


def load(path: Optional[str] = None):
    """Load liboracle_sgemm.so (or another build of oracle_sgemm.c at `path`),
    building the default one with gcc first if it is absent."""
    path = LIBRARY if path is None else path
    if path in _libs:
        return _libs[path]
    if path == LIBRARY and not os.path.exists(LIBRARY):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(path)
    f = lib.oracle_sgemm_f64
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_float,
                  ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                  ctypes.c_float, ctypes.c_void_p, ctypes.c_int64,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
    lib.oracle_default_threads.restype = ctypes.c_int
    lib.oracle_default_threads.argtypes = []
    _libs[path] = lib
    return lib


def oracle_threads() -> int:
    """Threads the oracle uses by default (all online cores)."""
    return int(load().oracle_default_threads())


@dataclasses.dataclass
class OracleResult:
    ref: np.ndarray      # float64 M x N: alpha*A@B + beta*C, unrounded
    sumabs: np.ndarray   # float64 M x N: sum_k |A[i][k]*B[k][j]|
    threads: int         # threads the oracle ran on


def _ptr(buf: Optional[np.ndarray]):
    if buf is None:
        return None
    if buf.dtype != np.float32:
        raise TypeError("oracle inputs must be float32")
    if not buf.flags["C_CONTIGUOUS"]:
        raise ValueError("oracle inputs must be C-contiguous buffers")
    return buf.ctypes.data


def _dims(buf, rows, cols, ld):
    if buf is not None and buf.ndim == 2:
        rows = buf.shape[0] if rows is None else rows
        cols = buf.shape[1] if cols is None else cols
        ld = buf.shape[1] if ld is None else ld
    return rows, cols, ld


def oracle_sgemm(A: Optional[np.ndarray], B: Optional[np.ndarray], C: Optional[np.ndarray],
                 alpha: float, beta: float,
                 M: Optional[int] = None, N: Optional[int] = None, K: Optional[int] = None,
                 lda: Optional[int] = None, ldb: Optional[int] = None, ldc: Optional[int] = None,
                 threads: int = 0, lib=None) -> OracleResult:
    """Reference GEMM on float32 row-major buffers.

    A, B, C are 2-D arrays (shape and stride inferred) or flat buffers with the
    sizes and leading dimensions given explicitly.  C is only read when
    beta != 0; A and B only when alpha != 0 and K > 0.
    """
    M, K, lda = _dims(A, M, K, lda)
    Kb, N, ldb = _dims(B, K, N, ldb)
    if K is None:
        K = Kb
    _, _, ldc = _dims(C, M, N, ldc)
    if None in (M, N, K):
        raise ValueError("sizes could not be inferred; pass M, N, K")
    lda = max(1, K) if lda is None else lda
    ldb = max(1, N) if ldb is None else ldb
    ldc = max(1, N) if ldc is None else ldc
    ref = np.empty((max(M, 0), max(N, 0)), dtype=np.float64)
    sumabs = np.empty_like(ref)
    lib = load() if lib is None else lib
    rc = lib.oracle_sgemm_f64(M, N, K, ctypes.c_float(alpha), _ptr(A), lda, _ptr(B), ldb,
                              ctypes.c_float(beta), _ptr(C), ldc,
                              ref.ctypes.data, sumabs.ctypes.data, int(threads))
    if rc < 0:
        raise ValueError(f"oracle_sgemm_f64 rejected argument {-rc}")
    return OracleResult(ref=ref, sumabs=sumabs, threads=int(rc))


def normalised_error(C_out: np.ndarray, res: OracleResult, C_in: Optional[np.ndarray],
                     alpha: float, beta: float, strict: bool = False) -> float:
    """Max normalised error of a float32 result against the oracle.

    C_out and C_in are M x N views (C_in is the C that was passed in; it is
    only used when beta != 0).  Returns +inf when an element whose
    denominator is zero is not exactly zero, or when C_out holds a NaN/inf
    where the reference is finite.
    """
    out = np.asarray(C_out, dtype=np.float64)
    ref = res.ref
    den = res.sumabs * (abs(alpha) if strict else 1.0)
    if beta != 0.0:
        den = den + np.abs(beta * np.asarray(C_in, dtype=np.float64))
    diff = np.abs(out - ref)
    if not np.all(np.isfinite(out[np.isfinite(ref)])):
        return float("inf")
    zero = den == 0.0
    if np.any(out[zero] != 0.0):
        return float("inf")
    if np.all(zero):
        return 0.0
    return float(np.max(diff[~zero] / den[~zero]))
