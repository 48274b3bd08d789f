"""hip_sgemm_ex_noalloc through the C ABI against hip_sgemm_ex: the same
plans and kernels with split K's workspace in the library's fixed device
array instead of the stream-ordered pool.  Outputs must equal
hip_sgemm_ex's bit for bit and the oracle within the 1e-5 bound, on two
split-K calls in a row (the second smaller, reusing the array the first
left behind), in every operand orientation, and on the plans without
workspace.
"""

from __future__ import annotations

import numpy as np
import pytest

from dense_fp32_matrix_row_amd import inputs, sgemm
from oracle import oracle
from tests import gpu_harness as gh

pytestmark = pytest.mark.gpu

BOUND = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _device():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    sgemm.load()


def _stored(X, trans):
    """The array the caller passes for op(X) = X (trans False) or X^T."""
    return np.ascontiguousarray(X.T) if trans else X


def _call(entry, ta, tb, A, B, C, alpha, beta):
    """One call of `entry` (hip_sgemm_ex or hip_sgemm_ex_noalloc) through
    the guarded harness; returns C_out."""
    M, K = A.shape
    N = B.shape[1]
    sa, sb = _stored(A, ta), _stored(B, tb)
    op_a, op_b = "T" if ta else "N", "T" if tb else "N"

    def run(M_, N_, K_, al, pa, lda, pb, ldb, be, pc, ldc, stream):
        return entry(op_a, op_b, M_, N_, K_, al, pa, lda, pb, ldb, be, pc, ldc, stream)

    # the harness lays out A and B as given (2-D arrays: M x K, K x N); the
    # stored transposes have the shapes K x M and N x K, with the leading
    # dimensions of those arrays
    case = gh.Case(M, N, K, alpha, beta, sa, sb, C, lda=sa.shape[1], ldb=sb.shape[1])
    out, st = gh.run(case, run)
    assert st == 0, sgemm.hip_sgemm_status_string(st)
    return out


def _check(M, N, K, ta, tb, seed, alpha=0.75, beta=-1.5):
    print(f"[noalloc] {M}x{N}x{K} op_a={'T' if ta else 'N'} op_b={'T' if tb else 'N'} "
          f"plan={sgemm.hip_sgemm_plan(M, N, K)['name']}", flush=True)
    A, B, C = inputs.make_abc(M, N, K, seed)
    want = _call(sgemm.hip_sgemm_ex, ta, tb, A, B, C, alpha, beta)
    got = _call(sgemm.hip_sgemm_ex_noalloc, ta, tb, A, B, C, alpha, beta)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    ref = oracle.oracle_sgemm(A, B, C, alpha, beta)
    err = oracle.normalised_error(got, ref, C, alpha, beta, strict=True)
    assert err <= BOUND, err


def test_noalloc_two_split_calls_in_a_row():
    """A split-K call, then a smaller one over the array the first left."""
    first, second = (700, 600, 8200), (512, 512, 4096)
    for shape in (first, second):
        assert sgemm.hip_sgemm_plan(*shape)["name"] == "split_k"
        assert sgemm.hip_sgemm_plan(*shape)["workspace_bytes"] <= sgemm.NOALLOC_WORKSPACE_BYTES
    _check(*first, False, False, 31001)
    _check(*second, False, False, 31002)


@pytest.mark.parametrize("ta,tb", [(False, True), (True, False), (True, True)])
def test_noalloc_split_every_orientation(ta, tb):
    _check(700, 600, 8200, ta, tb, 31010 + 2 * ta + tb)


@pytest.mark.parametrize("M,N,K", [(1024, 1024, 1024), (4097, 4097, 64), (2049, 2049, 64), (1025, 1025, 300),
                                   (300, 260, 500), (12, 3000, 2000), (3000, 7, 2000)])
def test_noalloc_plans_without_workspace(M, N, K):
    assert sgemm.hip_sgemm_plan(M, N, K)["workspace_bytes"] == 0
    _check(M, N, K, False, False, 31100 + M + N + K)


def test_workspace_follows_the_stream():
    """Split K on a stream of its own (not the null stream): the pool and
    the fixed array are those of the device the stream feeds, looked up
    from the stream; same bits as on the current stream."""
    import torch
    side = torch.cuda.Stream()
    shape = (700, 600, 8200)
    A, B, C = inputs.make_abc(*shape, 31200)
    print(f"[noalloc] {shape} on a side stream", flush=True)
    outs = {}
    for name, entry in (("pool", sgemm.hip_sgemm_ex), ("fixed", sgemm.hip_sgemm_ex_noalloc)):
        def on_side(M_, N_, K_, al, pa, lda, pb, ldb, be, pc, ldc, stream, entry=entry):
            torch.cuda.synchronize()  # the harness's copies are on the current stream
            return entry("N", "N", M_, N_, K_, al, pa, lda, pb, ldb, be, pc, ldc, side)
        out, st = gh.run(gh.Case(*shape, 0.75, -1.5, A, B, C), on_side)
        assert st == 0, sgemm.hip_sgemm_status_string(st)
        outs[name] = out
    want = _call(sgemm.hip_sgemm_ex, False, False, A, B, C, 0.75, -1.5)
    for out in outs.values():
        assert np.array_equal(out.view(np.uint32), want.view(np.uint32))


def test_noalloc_quick_returns_and_errors():
    """Argument errors and quick returns as hip_sgemm_ex (nothing launched
    for M == 0; C <- beta*C for K == 0)."""
    import torch
    dC = torch.full((4, 4), 2.0, device="cuda")
    assert sgemm.hip_sgemm_ex_noalloc("N", "N", 0, 4, 4, 1.0, None, 4, None, 4, 0.0, None, 4) == 0
    assert sgemm.hip_sgemm_ex_noalloc("N", "N", 4, 4, 0, 1.0, None, 1, None, 4, 3.0, dC, 4) == 0
    torch.cuda.synchronize()
    assert torch.all(dC == 6.0)
    assert sgemm.hip_sgemm_ex_noalloc("X", "N", 4, 4, 4, 1.0, dC, 4, dC, 4, 0.0, dC, 4) == \
        sgemm.STATUS_BAD_OP_A
