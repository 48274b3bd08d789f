"""Problems whose operands span more than 2^31 elements: every offset past the
32-bit range (a row of A or C times its leading dimension, a transposed A's
k times lda) has to be formed in 64 bits, on every plan that handles such a
shape.

The operands are drawn on the device from a seeded torch generator
(uniform[-1, 1), the test workloads' distribution) so that no multi-gigabyte
array passes through the host; sampled rows (both ends, the middle, the
rows whose offsets cross 2^31) are copied back and compared with the CPU
reference.  C is allocated with padding columns holding a sentinel that must
survive, so a wrapped 32-bit offset that lands outside the window is caught
as well as one that lands inside it.
"""

from __future__ import annotations

import numpy as np
import pytest

from dense_fp32_matrix_row_amd import sgemm
from oracle import oracle

pytestmark = pytest.mark.gpu

BOUND = 1e-5
SENTINEL = -7.25e30
PAD = 4  # padding columns of C


@pytest.fixture(scope="module", autouse=True)
def _device():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    sgemm.load()
    yield
    torch.cuda.empty_cache()


def _uniform(rows, cols, seed):
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    t = torch.empty(rows, cols, device="cuda")
    t.uniform_(-1.0, 1.0, generator=g)
    return t


def _padded_c(M, N, seed):
    """C (M x N) inside an M x (N + PAD) buffer whose padding holds SENTINEL."""
    import torch
    buf = torch.full((M, N + PAD), SENTINEL, device="cuda")
    buf[:, :N] = _uniform(M, N, seed)
    return buf


def _sample_rows(M):
    return sorted({0, 1, 255, 256, M // 2, M - 257, M - 2, M - 1})


def _check(call, A_rows, B, C0_rows, buf, rows, N, alpha, beta, what):
    st = call()
    assert st == 0, (what, sgemm.hip_sgemm_status_string(st))
    import torch
    torch.cuda.synchronize()
    got = buf[rows].cpu().numpy()
    assert np.all(got[:, N:] == np.float32(SENTINEL)), (what, "padding of C changed")
    ref = oracle.oracle_sgemm(A_rows, B, C0_rows, alpha, beta)
    err = oracle.normalised_error(got[:, :N], ref, C0_rows, alpha, beta, strict=True)
    assert err <= BOUND, (what, err)


def test_a_beyond_2_31_elements():
    """A is 65536 x 40000 (2.6e9 elements): row offsets row0 * lda exceed
    2^31 from row 53688 on (128 x 128 whole tiles under level 10)."""
    import torch
    M, N, K, alpha, beta = 65536, 128, 40000, 0.5, 2.0
    print(f"[large] A {M}x{K} ({M * K:.3g} elements), N={N}", flush=True)
    A = _uniform(M, K, 11)
    B = _uniform(K, N, 12)
    C0 = _padded_c(M, N, 13)
    buf = torch.empty_like(C0)
    rows = _sample_rows(M)
    A_rows = A[rows].cpu().numpy()
    B_h = B.cpu().numpy()
    C0_rows = C0[rows, :N].cpu().numpy()
    for level in (10, 9, None):
        buf.copy_(C0)

        def call(level=level):
            args = (M, N, K, alpha, A, K, B, N, beta, buf, N + PAD)
            return sgemm.hip_sgemm(*args) if level is None else sgemm.hip_sgemm_level(level, *args)
        print(f"[large] A beyond 2^31: level {level}", flush=True)
        _check(call, A_rows, B_h, C0_rows, buf, rows, N, alpha, beta, level)
    del A, B, C0, buf


def test_c_beyond_2_31_elements_every_level():
    """C is 46400 x 46400 (2.15e9 elements, beta = 1 reads it): row offsets
    row * ldc exceed 2^31 on the last rows, for every rung of the ladder."""
    import torch
    M = N = 46400
    K, alpha, beta = 32, 1.0, 1.0
    print(f"[large] C {M}x{N} ({M * N:.3g} elements), K={K}", flush=True)
    A = _uniform(M, K, 21)
    B = _uniform(K, N, 22)
    C0 = _padded_c(M, N, 23)
    buf = torch.empty_like(C0)
    rows = _sample_rows(M)
    A_rows = A[rows].cpu().numpy()
    B_h = B.cpu().numpy()
    C0_rows = C0[rows, :N].cpu().numpy()
    for level in range(sgemm.hip_sgemm_num_levels()):
        buf.copy_(C0)

        def call(level=level):
            return sgemm.hip_sgemm_level(level, M, N, K, alpha, A, K, B, N, beta, buf, N + PAD)
        print(f"[large] C beyond 2^31: level {level}", flush=True)
        _check(call, A_rows, B_h, C0_rows, buf, rows, N, alpha, beta, level)
    del A, B, C0, buf


def test_transposed_a_beyond_2_31_elements():
    """op(A) = A^T with A stored K x M = 40000 x 65536 (2.6e9 elements): the
    k * lda offsets of the transposed staging exceed 2^31."""
    import torch
    M, N, K, alpha, beta = 65536, 128, 40000, -1.5, 0.0
    print(f"[large] A^T stored {K}x{M} ({M * K:.3g} elements), N={N}", flush=True)
    At = _uniform(K, M, 31)
    B = _uniform(K, N, 32)
    buf = torch.full((M, N + PAD), float("nan"), device="cuda")
    buf[:, N:] = SENTINEL
    rows = _sample_rows(M)
    A_rows = np.ascontiguousarray(At[:, rows].cpu().numpy().T)
    B_h = B.cpu().numpy()

    def call():
        return sgemm.hip_sgemm_ex("T", "N", M, N, K, alpha, At, M, B, N, beta, buf, N + PAD)
    print("[large] transposed A beyond 2^31: level 10", flush=True)
    # beta = 0 with NaN in C: C must not be read
    _check(call, A_rows, B_h, None, buf, rows, N, alpha, beta, "A^T")
    del At, B, buf


@pytest.mark.parametrize("lda,launches", [(131000, 1), (131080, 3)])
def test_fringe_beside_the_tiles_near_2_31_bytes(lda, launches):
    """4097 x 4097 x 64 with A's rows lda apart: every block of the
    one-launch plan reads row M - 1 of A, 4096 lda floats past its first
    row.  At lda = 131000 that is just below 2^31 bytes and the one launch
    runs; at 131080 it is past, and the call falls back to the grid plus the
    thin kernels (three launches).  Either way row M - 1 and column N - 1
    must match the reference."""
    import torch
    M = N = 4097
    K, alpha, beta = 64, 0.5, 3.0
    assert (4096 * lda + K + 32) * 4 < 2 ** 31 if launches == 1 else 4096 * lda * 4 >= 2 ** 31
    print(f"[large] fringe beside the tiles, lda {lda} ({M * lda:.3g} elements)", flush=True)
    A = _uniform(M, lda, 41)
    B = _uniform(K, N, 42)
    C0 = _padded_c(M, N, 43)
    buf = C0.clone()
    rows = _sample_rows(M)
    A_rows = A[rows, :K].cpu().numpy()
    B_h = B.cpu().numpy()
    C0_rows = C0[rows, :N].cpu().numpy()

    def call():
        return sgemm.hip_sgemm(M, N, K, alpha, A, lda, B, N, beta, buf, N + PAD)
    _check(call, A_rows, B_h, C0_rows, buf, rows, N, alpha, beta, f"lda {lda}")
    del A, B, C0, buf
