"""Python binding of libsgemm (ctypes).  Argument marshalling only: every
operation runs in the library's HIP kernels; there is no fallback.

The functions carry the C ABI's names and argument order (include/sgemm.h).
Matrix arguments accept a torch device tensor (its data_ptr() is passed), an
integer device address, or None (NULL).  `stream` accepts None (torch's
current stream on the current device), a torch.cuda.Stream, or an integer
hipStream_t handle (0 = the null stream).

torch is imported before the library is loaded: torch ships its own HIP
runtime (libamdhip64.so.7) and the library must bind to that same runtime,
so that device pointers and stream handles from torch are valid for it.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(HERE, "libsgemm.so")

STATUS_UNKNOWN_LEVEL = -100
STATUS_UNKNOWN_CONFIG = -101
STATUS_BAD_OP_A = -102
STATUS_BAD_OP_B = -103
STATUS_WORKSPACE_LIMIT = -104
NOALLOC_WORKSPACE_BYTES = 8 << 20  # SGEMM_NOALLOC_WORKSPACE_BYTES

# Every exported symbol of include/sgemm.h.
EXPORTS = (
    "hip_sgemm", "hip_sgemm_level", "hip_sgemm_num_levels", "hip_sgemm_level_name",
    "hip_sgemm_status_string", "hip_sgemm_auto_level", "hip_sgemm_launch_shape",
    "hip_sgemm_tile_split", "hip_sgemm_num_tiles", "hip_sgemm_tile_name", "hip_sgemm_ex",
    "hip_sgemm_plan", "hip_sgemm_ex_noalloc",
)

# Plan ids of hip_sgemm_plan (SGEMM_PLAN_* in sgemm.h).
PLAN_NAMES = {0: "none", 1: "scale", 2: "few_rows", 3: "few_cols", 4: "tiles",
              5: "tiles_fringe", 6: "split_k", 7: "thin_panels"}

_lib = None


class SgemmError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"libsgemm status {status}: {message}")
        self.status = status


def load(path: Optional[str] = None):
    """Load libsgemm.so (built by dense_fp32_matrix_row_amd.build), or the
    build at `path`, which then serves every call of this module.  Raises if
    it is missing: there is no other implementation to fall back on."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    import torch  # noqa: F401  (binds the library to torch's HIP runtime)
    path = LIBRARY if path is None else path
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m dense_fp32_matrix_row_amd.build` "
                           "or __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    fptr, vp, i32, f32 = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    gemm_args = [i32, i32, i32, f32, vp, i32, vp, i32, f32, vp, i32, vp]
    lib.hip_sgemm.restype = i32
    lib.hip_sgemm.argtypes = gemm_args
    lib.hip_sgemm_level.restype = i32
    lib.hip_sgemm_level.argtypes = [i32] + gemm_args
    lib.hip_sgemm_ex.restype = i32
    lib.hip_sgemm_ex.argtypes = [i32, i32] + gemm_args
    lib.hip_sgemm_ex_noalloc.restype = i32
    lib.hip_sgemm_ex_noalloc.argtypes = [i32, i32] + gemm_args
    lib.hip_sgemm_tile_split.restype = i32
    lib.hip_sgemm_tile_split.argtypes = [i32, i32] + gemm_args
    lib.hip_sgemm_num_tiles.restype = i32
    lib.hip_sgemm_num_tiles.argtypes = []
    lib.hip_sgemm_tile_name.restype = ctypes.c_char_p
    lib.hip_sgemm_tile_name.argtypes = [i32]
    lib.hip_sgemm_num_levels.restype = i32
    lib.hip_sgemm_num_levels.argtypes = []
    lib.hip_sgemm_level_name.restype = ctypes.c_char_p
    lib.hip_sgemm_level_name.argtypes = [i32]
    lib.hip_sgemm_status_string.restype = ctypes.c_char_p
    lib.hip_sgemm_status_string.argtypes = [i32]
    lib.hip_sgemm_auto_level.restype = i32
    lib.hip_sgemm_auto_level.argtypes = [i32, i32, i32, vp, i32, vp, i32, vp, i32]
    lib.hip_sgemm_launch_shape.restype = i32
    lib.hip_sgemm_launch_shape.argtypes = [i32, i32, i32, i32,
                                           ctypes.POINTER(ctypes.c_longlong), ctypes.POINTER(i32),
                                           ctypes.POINTER(ctypes.c_longlong), ctypes.POINTER(i32),
                                           ctypes.POINTER(i32)]
    lib.hip_sgemm_plan.restype = i32
    lib.hip_sgemm_plan.argtypes = [i32, i32, i32, ctypes.POINTER(i32), ctypes.POINTER(i32),
                                   ctypes.POINTER(ctypes.c_longlong)]
    del fptr
    _lib = lib
    return lib


def _addr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    dp = getattr(x, "data_ptr", None)
    if dp is None:
        raise TypeError(f"expected a tensor, an int address or None, got {type(x).__name__}")
    if getattr(x, "is_cuda", True) is False:
        raise TypeError("matrix tensors must live on the GPU")
    return int(dp())


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        if not torch.cuda.is_available():
            return None
        return int(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return stream
    handle = getattr(stream, "cuda_stream", None)
    if handle is None:
        raise TypeError("stream must be None, an int handle or a torch.cuda.Stream")
    return int(handle)


def hip_sgemm(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=None) -> int:
    """C <- alpha*A@B + beta*C with the library's choice of kernel; returns the
    status code (0 = enqueued)."""
    return int(load().hip_sgemm(int(M), int(N), int(K), float(alpha), _addr(A), int(lda),
                                _addr(B), int(ldb), float(beta), _addr(C), int(ldc),
                                _stream(stream)))


def hip_sgemm_level(level, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=None) -> int:
    """Same as hip_sgemm with the ladder rung `level` forced."""
    return int(load().hip_sgemm_level(int(level), int(M), int(N), int(K), float(alpha), _addr(A),
                                      int(lda), _addr(B), int(ldb), float(beta), _addr(C),
                                      int(ldc), _stream(stream)))


def _op(op) -> int:
    if isinstance(op, str):
        if len(op) != 1:
            raise ValueError(f"op must be one character, got {op!r}")
        return ord(op)
    return int(op)


def hip_sgemm_ex(op_a, op_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=None) -> int:
    """C <- alpha*op(A)@op(B) + beta*C; op_a / op_b are 'N' or 'T' (or 0 / 1)."""
    return int(load().hip_sgemm_ex(_op(op_a), _op(op_b), int(M), int(N), int(K), float(alpha),
                                   _addr(A), int(lda), _addr(B), int(ldb), float(beta), _addr(C),
                                   int(ldc), _stream(stream)))


def hip_sgemm_ex_noalloc(op_a, op_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                         stream=None) -> int:
    """hip_sgemm_ex with split K's workspace in the library's fixed device
    array: no allocation; overlapping calls on one GPU race."""
    return int(load().hip_sgemm_ex_noalloc(_op(op_a), _op(op_b), int(M), int(N), int(K),
                                           float(alpha), _addr(A), int(lda), _addr(B), int(ldb),
                                           float(beta), _addr(C), int(ldc), _stream(stream)))


def hip_sgemm_tile_split(tile, splits, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                         stream=None) -> int:
    """Level 9's kernel with tile shape `tile` and K cut into `splits` slices."""
    return int(load().hip_sgemm_tile_split(int(tile), int(splits), int(M), int(N), int(K),
                                           float(alpha), _addr(A), int(lda), _addr(B), int(ldb),
                                           float(beta), _addr(C), int(ldc), _stream(stream)))


def hip_sgemm_num_tiles() -> int:
    return int(load().hip_sgemm_num_tiles())


def hip_sgemm_tile_name(tile) -> Optional[str]:
    s = load().hip_sgemm_tile_name(int(tile))
    return None if s is None else s.decode()


def hip_sgemm_num_levels() -> int:
    return int(load().hip_sgemm_num_levels())


def hip_sgemm_level_name(level) -> Optional[str]:
    s = load().hip_sgemm_level_name(int(level))
    return None if s is None else s.decode()


def hip_sgemm_status_string(status) -> str:
    return load().hip_sgemm_status_string(int(status)).decode()


def hip_sgemm_auto_level(M, N, K, A, lda, B, ldb, C, ldc) -> int:
    return int(load().hip_sgemm_auto_level(int(M), int(N), int(K), _addr(A), int(lda), _addr(B),
                                           int(ldb), _addr(C), int(ldc)))


def hip_sgemm_launch_shape(level, M, N, K) -> dict:
    """Launch geometry of a level for a shape (nothing is launched)."""
    wg, kst = ctypes.c_longlong(), ctypes.c_longlong()
    thr, tm, tn = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    rc = load().hip_sgemm_launch_shape(int(level), int(M), int(N), int(K), ctypes.byref(wg),
                                       ctypes.byref(thr), ctypes.byref(kst), ctypes.byref(tm),
                                       ctypes.byref(tn))
    if rc != 0:
        raise SgemmError(rc, hip_sgemm_status_string(rc))
    return {"workgroups": wg.value, "threads": thr.value, "k_steps": kst.value,
            "tile_m": tm.value, "tile_n": tn.value}


def hip_sgemm_plan(M, N, K) -> dict:
    """The plan hip_sgemm takes for a shape: plan id and name, kernels per
    call, split-K workspace bytes (nothing is launched)."""
    plan, launches, ws = ctypes.c_int(), ctypes.c_int(), ctypes.c_longlong()
    rc = load().hip_sgemm_plan(int(M), int(N), int(K), ctypes.byref(plan), ctypes.byref(launches),
                               ctypes.byref(ws))
    if rc != 0:
        raise SgemmError(rc, hip_sgemm_status_string(rc))
    return {"plan": plan.value, "name": PLAN_NAMES[plan.value], "launches": launches.value,
            "workspace_bytes": ws.value}


def check(status: int) -> None:
    """Raise SgemmError for a non-zero status."""
    if status != 0:
        raise SgemmError(status, hip_sgemm_status_string(status))


def sgemm(A, B, C, alpha: float = 1.0, beta: float = 0.0, level: Optional[int] = None,
          stream=None) -> None:
    """Convenience form on 2-D row-major torch float32 device tensors whose
    rows may be strided (column stride 1): C <- alpha*A@B + beta*C."""
    for name, t in (("A", A), ("B", B), ("C", C)):
        if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
            raise ValueError(f"{name} must be a 2-D row-major view with unit column stride")
    M, K = A.shape
    K2, N = B.shape
    if K2 != K or tuple(C.shape) != (M, N):
        raise ValueError(f"shape mismatch: A {tuple(A.shape)}, B {tuple(B.shape)}, C {tuple(C.shape)}")
    lda, ldb, ldc = (max(t.stride(0), t.shape[1], 1) for t in (A, B, C))
    if level is None:
        rc = hip_sgemm(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream)
    else:
        rc = hip_sgemm_level(level, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream)
    check(rc)
