"""Non-finite inputs: +inf, -inf and NaN planted in A, B and C travel into C
exactly as the definition says, C = alpha * sum_k A[i][k] * B[k][j] +
beta * C[i][j] evaluated in IEEE arithmetic (an infinity times a nonzero
finite value is an infinity of the product's sign, inf + -inf and anything
with NaN is NaN, beta = 0 never reads C).  The CPU reference evaluates the
same sums in float64, so the pattern of NaNs and signed infinities of its
result is the expected one whatever the summation order; every finite
element must still meet the normalised-error bound.

An infinity in row i1 of A reaches every output of row i1, one in column
j2 of B every output of column j2, a NaN in row i3 of A the whole row: so a
kernel that pairs the wrong elements of A and B, or lets a zero-filled
edge meet a planted value, shows up as a wrong row or column of the
pattern.  The plants sit in the last row and column (the fringes and edge
tiles) and at the first and last k.  Run on every plan of level 10 and on
every rung of the ladder.
"""

from __future__ import annotations

import numpy as np
import pytest

from dense_fp32_matrix_row_amd import inputs, sgemm
from oracle import oracle
from tests import gpu_harness as gh

pytestmark = pytest.mark.gpu

BOUND = 1e-5


@pytest.fixture(scope="session", autouse=True)
def _device():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    sgemm.load()


def planted(M, N, K, seed):
    """Uniform[-1, 1] operands with +inf at A[M-1][0], -inf at B[K-1][N-1],
    NaN at A[M // 2][K // 2] (when M > 1) and +inf at C[0][N // 2]."""
    A, B, C = inputs.make_abc(M, N, K, seed)
    A[M - 1, 0] = np.inf
    B[K - 1, N - 1] = -np.inf
    if M > 1:
        A[M // 2, K // 2] = np.nan
    C[0, N // 2] = np.inf
    return A, B, C


def check(out, A, B, C, alpha, beta, what):
    res = oracle.oracle_sgemm(A, B, C, alpha, beta)
    ref = res.ref
    # the pattern: NaN where the reference is NaN, the same signed infinity
    # where it is infinite, finite elsewhere
    assert np.array_equal(np.isnan(out), np.isnan(ref)), (what, "NaN pattern")
    inf_ref = np.isinf(ref)
    assert np.array_equal(np.isinf(out), inf_ref), (what, "infinity pattern")
    assert np.array_equal(np.sign(out[inf_ref]), np.sign(ref[inf_ref])), (what, "infinity signs")
    # the planted values do reach something, so the pattern is not vacuous
    assert (~np.isfinite(ref)).any()
    fin = np.isfinite(ref)
    if fin.any():
        sub = oracle.OracleResult(ref=ref[fin], sumabs=res.sumabs[fin], threads=res.threads)
        err = oracle.normalised_error(out[fin], sub, C[fin], alpha, beta, strict=True)
        assert err <= BOUND, (what, err)


# (M, N, K, plan hip_sgemm_plan names): one shape per plan of level 10
PLANS = [
    (4097, 4097, 40, "tiles_fringe"),
    (1025, 1025, 200, "tiles_fringe"),
    (4096, 4096, 36, "tiles"),
    (2048, 2048, 100, "tiles"),
    (1000, 1000, 300, "tiles"),
    (2051, 2055, 300, "tiles_fringe"),
    (512, 512, 8192, "split_k"),
    (700, 600, 8200, "split_k"),
    (300, 260, 500, "thin_panels"),
    (1, 3001, 503, "few_rows"),
    (5, 3001, 503, "few_rows"),
    (16, 1000, 777, "few_rows"),
    (1500, 1, 503, "few_cols"),
    (1500, 7, 503, "few_cols"),
]


@pytest.mark.parametrize("M,N,K,plan", PLANS, ids=[f"{p[3]}-{p[0]}x{p[1]}x{p[2]}" for p in PLANS])
def test_nonfinite_every_plan(M, N, K, plan):
    print(f"[nonfinite] {M}x{N}x{K} {plan}", flush=True)
    assert sgemm.hip_sgemm_plan(M, N, K)["name"] == plan
    A, B, C = planted(M, N, K, 11000 + M + N + K)
    for alpha, beta in [(0.5, 3.0), (-1.0, 0.0)]:
        out, st = gh.run(gh.Case(M, N, K, alpha, beta, A, B, C), None)
        assert st == 0, sgemm.hip_sgemm_status_string(st)
        check(out, A, B, C, alpha, beta, (M, N, K, plan, alpha, beta))


@pytest.mark.parametrize("level", range(10))
def test_nonfinite_every_rung(level):
    M, N, K = 261, 133, 150
    print(f"[nonfinite] level {level} {M}x{N}x{K}", flush=True)
    A, B, C = planted(M, N, K, 11500 + level)
    for alpha, beta in [(0.5, 3.0), (-1.0, 0.0)]:
        out, st = gh.run(gh.Case(M, N, K, alpha, beta, A, B, C), level)
        assert st == 0, sgemm.hip_sgemm_status_string(st)
        check(out, A, B, C, alpha, beta, (level, alpha, beta))
