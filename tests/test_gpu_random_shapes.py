"""Seeded random problems through hip_sgemm_ex, every element against the
CPU reference: problems of every plan the dispatcher has (thin sides of
1-16, small problems, tile grids sized around the tiles' multiples -- a
multiple of 64, 128 or 256, or one to seventeen off it --, grids one row
and / or column past a multiple, deep K over small grids), all four
operand orientations, padded leading dimensions, bases offset
by one to three elements, and alpha / beta including beta = 0 over a C full
of NaN; and, for every forced rung of the ladder (levels 0-9), medium
shapes with partial block tiles, ragged K, padded strides and offsets.  The
guarded harness also checks that nothing outside C's window changes.  The
draws are fixed by the seed, so a failure names its case.
"""

from __future__ import annotations

import numpy as np
import pytest

from dense_fp32_matrix_row_amd import inputs, sgemm
from oracle import oracle
from tests import gpu_harness as gh

pytestmark = pytest.mark.gpu

BOUND = 1e-5
CASES = 160
MAX_WORK = 4e9  # M * N * K per case, so the reference stays quick


@pytest.fixture(scope="module", autouse=True)
def _device():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    sgemm.load()


def _near(rng, tiles_hi: int) -> int:
    """A multiple of 64, 128 or 256, or a few off it."""
    base = int(rng.choice([64, 128, 256])) * int(rng.integers(1, tiles_hi + 1))
    return max(1, base + int(rng.choice([0, 0, 1, -1, 2, 15, 16, 17, -15])))


def _draw(rng):
    """One problem of a kind picked first, so that every plan of the
    dispatcher gets its share: thin, small (16-row panels), a tile grid, a
    grid missing a tile multiple by one row and / or column, split K."""
    while True:
        kind = rng.choice(["thin", "small", "tiles", "fringe", "split"], p=[0.15, 0.15, 0.4, 0.15, 0.15])
        if kind == "thin":
            M, N = int(rng.integers(1, 17)), int(rng.integers(17, 4000))
            if rng.random() < 0.5:
                M, N = N, M
            K = int(rng.integers(1, 6000))
        elif kind == "small":
            M, N, K = (int(v) for v in rng.integers(17, 500, 3))
        elif kind == "tiles":
            M, N = _near(rng, 16), _near(rng, 16)
            K = int(rng.choice([1, 3, 16, 17, 64, 65, 300, 1000, 2047]))
        elif kind == "fringe":
            tile = int(rng.choice([64, 128, 256]))
            M = tile * int(rng.integers(8, 17)) + int(rng.integers(0, 2))
            N = tile * int(rng.integers(8, 17)) + int(rng.integers(0, 2))
            K = int(rng.choice([5, 16, 33, 100, 257]))
        else:
            M, N = (int(v) for v in rng.integers(400, 1000, 2))
            K = int(rng.integers(4096, 9000))
        if M * N * K <= MAX_WORK:
            break
    ta, tb = bool(rng.integers(0, 2)), bool(rng.integers(0, 2))
    alpha = float(rng.choice([1.0, -1.5, 0.5]))
    beta = float(rng.choice([0.0, 1.0, -2.0]))
    pads = tuple(int(v) for v in rng.integers(0, 6, 3))
    offs = tuple(int(v) for v in rng.integers(0, 4, 3))
    return M, N, K, ta, tb, alpha, beta, pads, offs


def _cases():
    rng = np.random.default_rng(20261202)
    return [_draw(rng) for _ in range(CASES)]


@pytest.mark.parametrize("case", range(CASES))
def test_random_problem_matches_reference(case):
    M, N, K, ta, tb, alpha, beta, pads, offs = _cases()[case]
    plan = sgemm.hip_sgemm_plan(M, N, K)["name"]
    print(f"[random {case}] {M}x{N}x{K} op_a={'T' if ta else 'N'} op_b={'T' if tb else 'N'} "
          f"alpha={alpha} beta={beta} pads={pads} offs={offs} plan={plan}", flush=True)
    A, B, C = inputs.make_abc(M, N, K, 40000 + case)
    if beta == 0.0:
        C = np.full_like(C, np.nan)  # must not be read
    sa = np.ascontiguousarray(A.T) if ta else A
    sb = np.ascontiguousarray(B.T) if tb else B
    op_a, op_b = ("T" if ta else "N"), ("T" if tb else "N")

    def call(M_, N_, K_, al, pa, lda, pb, ldb, be, pc, ldc, stream):
        return sgemm.hip_sgemm_ex(op_a, op_b, M_, N_, K_, al, pa, lda, pb, ldb, be, pc, ldc, stream)

    c = gh.Case(M, N, K, alpha, beta, sa, sb, C, lda=sa.shape[1] + pads[0],
                ldb=sb.shape[1] + pads[1], ldc=N + pads[2], a_off=offs[0], b_off=offs[1],
                c_off=offs[2])
    out, st = gh.run(c, call)
    assert st == 0, sgemm.hip_sgemm_status_string(st)
    ref = oracle.oracle_sgemm(A, B, C, alpha, beta)
    err = oracle.normalised_error(out, ref, C, alpha, beta, strict=True)
    assert err <= BOUND, (case, M, N, K, ta, tb, err)


RUNG_CASES = 8


def _rung_cases(level):
    """Medium shapes for a forced rung: partial block tiles of every size
    the rungs use (up to 256 x 128), ragged K, padded strides, offsets."""
    rng = np.random.default_rng(20261203 + level)
    out = []
    for _ in range(RUNG_CASES):
        M, N = (int(v) for v in rng.integers(100, 700, 2))
        K = int(rng.integers(1, 600))
        alpha = float(rng.choice([1.0, -1.5, 0.5]))
        beta = float(rng.choice([0.0, 1.0, -2.0]))
        pads = tuple(int(v) for v in rng.integers(0, 6, 3))
        offs = tuple(int(v) for v in rng.integers(0, 4, 3))
        out.append((M, N, K, alpha, beta, pads, offs))
    return out


@pytest.mark.parametrize("level", range(10))
def test_random_problems_every_rung(level):
    print(f"[random rung] level {level}", flush=True)
    for i, (M, N, K, alpha, beta, pads, offs) in enumerate(_rung_cases(level)):
        A, B, C = inputs.make_abc(M, N, K, 41000 + 10 * level + i)
        if beta == 0.0:
            C = np.full_like(C, np.nan)  # must not be read
        c = gh.Case(M, N, K, alpha, beta, A, B, C, lda=K + pads[0], ldb=N + pads[1], ldc=N + pads[2],
                    a_off=offs[0], b_off=offs[1], c_off=offs[2])
        out, st = gh.run(c, level)
        assert st == 0, sgemm.hip_sgemm_status_string(st)
        ref = oracle.oracle_sgemm(A, B, C, alpha, beta)
        err = oracle.normalised_error(out, ref, C, alpha, beta, strict=True)
        assert err <= BOUND, (level, i, M, N, K, pads, offs, err)
