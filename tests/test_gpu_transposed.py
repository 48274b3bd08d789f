"""hip_sgemm_ex with op(A), op(B) in {N, T} through the C ABI: every level-10
plan (thin rows / columns, whole-tile grid + fringe, ragged K, two-slice
tiles, split K) in all four orientations against the CPU reference, with
padded and misaligned storage and guard regions around C.

The tile kernels stage either orientation into the same k-major LDS layout,
and the thin kernels keep the same per-lane k order, so wherever the plan is
the same for every orientation the transposed calls must reproduce the
untransposed result bit for bit.  Where it is not, the expected identities
are narrower: the vector-ALU few-columns kernel reads A by rows, so one to
four columns with A stored transposed take the matrix-core thin form (B's
orientation never changes the plan there).
"""

from __future__ import annotations

import numpy as np
import pytest

from dense_fp32_matrix_row_amd import inputs, sgemm
from oracle import oracle
from tests import gpu_harness as gh

pytestmark = pytest.mark.gpu

BOUND = 1e-5
OPS = [("N", "N"), ("N", "T"), ("T", "N"), ("T", "T")]


@pytest.fixture(scope="session", autouse=True)
def _device():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    sgemm.load()


def run_ex(op_a, op_b, A, B, C, alpha, beta, pads=(0, 0, 0), offs=(0, 0, 0)):
    """A (M x K) and B (K x N) are the logical operands; they are stored as
    given by op_a / op_b (transposed copies for 'T') with row padding."""
    M, K = A.shape
    N = B.shape[1]
    sa = np.ascontiguousarray(A.T) if op_a == "T" else A
    sb = np.ascontiguousarray(B.T) if op_b == "T" else B
    lda = max(1, sa.shape[1]) + pads[0]
    ldb = max(1, sb.shape[1]) + pads[1]
    ldc = max(1, N) + pads[2]
    case = gh.Case(M, N, K, alpha, beta, sa, sb, C, lda, ldb, ldc, *offs)
    return gh.run(case, lambda *args: sgemm.hip_sgemm_ex(op_a, op_b, *args))


# (M, N, K, plan, which results must be bit-identical: "all" four, "b" =
# B's orientation does not matter)
SHAPES = [
    (5, 3001, 777, "few rows", "all"),
    (1, 4097, 4097, "one row on the vector ALUs: whole sweeps, K tail, edge block", "all"),
    (2, 1000, 2049, "two rows on the vector ALUs: whole sweeps, K tail", "all"),
    (3, 3001, 2300, "three rows on the vector ALUs: whole sweeps, K tail, edge block", "all"),
    (4097, 1, 4097, "one column on the vector ALUs (A^T: matrix-core thin form)", "b"),
    (2500, 3, 2300, "three columns on the vector ALUs, whole and partial chunks", "b"),
    (16, 1000, 333, "sixteen rows", "all"),
    (1500, 7, 2003, "few columns", "all"),
    (1500, 3, 2003, "three columns (A^T: matrix-core thin form)", "b"),
    (2051, 2055, 300, "128x128 grid + fringe", "all"),
    (4096 + 3, 4096 + 16, 40, "256x128 grid + fringe", "all"),
    (4097, 4097, 70, "256x128 grid, one row and one column in the tiles' launch", "all"),
    (4097, 4096, 17, "256x128 grid, one row in the tiles' launch", "all"),
    (4096, 4097, 5, "256x128 grid, one column in the tiles' launch, K below a stage", "all"),
    (2049, 2049, 70, "128x128 grid, one row and one column in the tiles' launch", "all"),
    (1025, 1025, 130, "64x64 grid, one row and one column in the tiles' launch", "all"),
    (1025, 4097, 37, "128x128 grid of 8 tile rows (shares of 16 columns), fringe in the tiles' launch", "all"),
    (2561, 6145, 37, "256x128 grid, uneven shares (13 columns, 6 rows), fringe in the tiles' launch", "all"),
    (1025, 3073, 65, "64x64 grid of 16 x 48 tiles (shares of 4 columns, 2 rows), fringe in the tiles' launch", "all"),
    (3073, 1024, 65, "64x64 grid of 48 x 16 tiles, one row in the tiles' launch", "all"),
    (8192, 8, 1000, "eight columns, two per lane", "all"),
    (16, 16384, 777, "sixteen rows, two columns per lane", "all"),
    (2048, 2048, 100, "128x128 grid, K ragged", "all"),
    (4096, 4096, 36, "256x128 grid, K ragged", "all"),
    (1000, 1000, 300, "64x64 loop tiles, edges", "all"),
    (1024, 1024, 4096, "64x64 loop tiles, deep K", "all"),
    (512, 512, 8192, "split K, 64x64 loop tiles, 8 slices", "all"),
    (700, 600, 8200, "split K, 64x64 edge tiles, ragged K", "all"),
    (100, 3000, 2100, "split K, wide shallow grid, 2 slices, ragged K", "all"),
    (4200, 60, 2500, "split K, tall narrow grid, 2 slices, ragged K", "all"),
    (300, 260, 5000, "16-row panels, deep K", "all"),
    (17, 33, 65, "odd", "all"),
    (129, 65, 31, "odd", "all"),
]


@pytest.mark.parametrize("M,N,K,plan,same", SHAPES, ids=[f"{s[0]}x{s[1]}x{s[2]}" for s in SHAPES])
def test_transposed_operands(M, N, K, plan, same):
    print(f"[transposed] {M}x{N}x{K}: {plan}", flush=True)
    A, B, C = inputs.make_abc(M, N, K, 5100 + M + N + K)
    ref = oracle.oracle_sgemm(A, B, C, 0.5, 3.0)
    outs = {}
    for op_a, op_b in OPS:
        out, st = run_ex(op_a, op_b, A, B, C, 0.5, 3.0)
        assert st == 0, (op_a, op_b, sgemm.hip_sgemm_status_string(st))
        err = oracle.normalised_error(out, ref, C, 0.5, 3.0, strict=True)
        assert err <= BOUND, (op_a, op_b, err)
        outs[op_a + op_b] = out
    groups = {"all": [("NN", "NT", "TN", "TT")], "b": [("NN", "NT"), ("TN", "TT")]}[same]
    for group in groups:
        for key in group[1:]:
            assert np.array_equal(outs[group[0]].view(np.uint32), outs[key].view(np.uint32)), (group[0], key)


@pytest.mark.parametrize("M,N,K", [(131, 257, 515), (7, 1029, 301), (1029, 9, 301), (2051, 2053, 64),
                                   (4097, 4097, 40), (2049, 2049, 40), (1025, 1025, 77)])
def test_transposed_padded_misaligned(M, N, K):
    """Row padding that breaks 16-byte alignment of rows and bases that are
    only 4-byte aligned, beta = 0 with NaN in C (C must not be read)."""
    print(f"[transposed alignment] {M}x{N}x{K}", flush=True)
    A, B, _ = inputs.make_abc(M, N, K, 5200 + M)
    nanC = np.full((M, N), np.nan, np.float32)
    ref = oracle.oracle_sgemm(A, B, None, -1.5, 0.0)
    for op_a, op_b in OPS:
        out, st = run_ex(op_a, op_b, A, B, nanC, -1.5, 0.0, pads=(3, 5, 7), offs=(1, 2, 3))
        assert st == 0 and np.all(np.isfinite(out)), (op_a, op_b)
        assert oracle.normalised_error(out, ref, None, -1.5, 0.0, strict=True) <= BOUND, (op_a, op_b)


@pytest.mark.parametrize("M,N,K", [(4097, 4097, 33), (2049, 2049, 33), (1025, 1025, 200), (520, 390, 3000),
                                   (3, 2000, 999), (4, 3001, 2300), (2500, 2, 2300)])
def test_transposed_integer_exact(M, N, K):
    """Integer entries: every orientation equals the reference bit for bit."""
    print(f"[transposed integer] {M}x{N}x{K}", flush=True)
    A, B, C = inputs.integer_abc(M, N, K, seed=5300 + K)
    ref = oracle.oracle_sgemm(A, B, C, 2.0, -1.0)
    for op_a, op_b in OPS:
        out, st = run_ex(op_a, op_b, A, B, C, 2.0, -1.0)
        assert st == 0
        assert np.array_equal(out.astype(np.float64), ref.ref), (op_a, op_b)


def test_transposed_quick_returns():
    """alpha = 0 and K = 0 give C = beta*C without reading A or B (NaN here)."""
    M, N, K = 70, 90, 50
    rng = np.random.default_rng(5400)
    C = inputs.uniform_f32(rng, (M, N))
    nanA = np.full((M, K), np.nan, np.float32)
    nanB = np.full((K, N), np.nan, np.float32)
    for op_a, op_b in OPS:
        out, st = run_ex(op_a, op_b, nanA, nanB, C, 0.0, 3.0)
        assert st == 0 and np.array_equal(out, np.float32(3.0) * C)
