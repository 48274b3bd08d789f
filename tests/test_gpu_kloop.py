"""Level 10's 256 x 128 whole-tile kernel with the K loop in assembly
(l10_kloop.hip) through the C ABI: K step counts that exercise each path of
the loop (one step, pairs only, pairs plus the odd step, long loops), a
ragged first stage (K % 16 != 0), a fringe around the whole-tile grid,
padded and 4-byte-aligned storage, beta = 0 over NaN, integer data
(bit-exact against the reference), the tile-forcing entry point on grids
too small for the dispatch rule, and bit-identity with level 9's compiled
loop on the same tile when K % 16 == 0.
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


# (M, N, K, what): all have at least 512 whole 256 x 128 tiles, so level 10
# takes the assembly loop for the grid
SHAPES = [
    (4096, 4096, 16, "one K step (no pair)"),
    (4096, 4096, 32, "one pair"),
    (4096, 4096, 48, "pair + odd step"),
    (4096, 4096, 272, "8 pairs + odd step"),
    (8192, 2048, 1024, "64 K-step pairs, 8192 rows"),
    (4096 + 5, 4096 + 9, 80, "grid + 5-row / 9-column fringe"),
    (4096, 4096, 5, "K = 5: one ragged stage"),
    (4096, 4096, 21, "ragged stage + one whole stage"),
    (4096, 4096, 1001, "ragged stage (9) + 62 whole stages"),
    (4096 + 1, 4096 + 1, 4097, "4097^3: ragged stage (1) + 256 whole stages, fringe"),
]


@pytest.mark.parametrize("M,N,K,what", SHAPES, ids=[s[3] for s in SHAPES])
def test_kloop_matches_reference(M, N, K, what):
    print(f"[kloop] {M}x{N}x{K}: {what}", flush=True)
    A, B, C = inputs.make_abc(M, N, K, 12000 + M + N + K)
    for alpha, beta in [(0.5, 3.0), (1.0, 0.0)]:
        out, st = gh.run(gh.Case(M, N, K, alpha, beta, A, B, C), 10)
        assert st == 0, sgemm.hip_sgemm_status_string(st)
        ref = oracle.oracle_sgemm(A, B, C, alpha, beta)
        err = oracle.normalised_error(out, ref, C, alpha, beta, strict=True)
        assert err <= BOUND, (alpha, beta, err)


def test_kloop_padded_misaligned_nan_c():
    """lda = K + 3, ldb = N + 5, ldc = N + 7 and bases 4, 8, 12 bytes past a
    16-byte boundary: every 128-bit load and store is misaligned; beta = 0
    with NaN in C (C must not be read)."""
    M, N, K = 4096, 4096, 64
    print(f"[kloop alignment] {M}x{N}x{K}", flush=True)
    A, B, _ = inputs.make_abc(M, N, K, 12500)
    nanC = np.full((M, N), np.nan, np.float32)
    out, st = gh.run(gh.Case(M, N, K, -1.5, 0.0, A, B, nanC, K + 3, N + 5, N + 7, 1, 2, 3), 10)
    assert st == 0 and np.all(np.isfinite(out))
    ref = oracle.oracle_sgemm(A, B, None, -1.5, 0.0)
    assert oracle.normalised_error(out, ref, None, -1.5, 0.0, strict=True) <= BOUND


def test_kloop_integer_exact():
    """Integer entries: every sum is exact in any order, so all of C must
    equal the reference bit for bit (every tile, lane and register)."""
    M, N, K = 4096, 4096, 48
    print(f"[kloop integer] {M}x{N}x{K}", flush=True)
    A, B, C = inputs.integer_abc(M, N, K, seed=12600)
    out, st = gh.run(gh.Case(M, N, K, 2.0, -1.0, A, B, C), 10)
    assert st == 0
    assert np.array_equal(out.astype(np.float64), oracle.oracle_sgemm(A, B, C, 2.0, -1.0).ref)


@pytest.mark.parametrize("K", [48, 1040])
def test_kloop_bit_identical_to_level9(K):
    """Level 9 runs the same 256 x 128 tile with the compiled K loop: same
    blocks, same operands per MFMA, same k order, so the same bits."""
    M = N = 4096
    print(f"[kloop vs level 9] {M}x{N}x{K}", flush=True)
    A, B, C = inputs.make_abc(M, N, K, 12700 + K)
    res = gh.Resident(A, B, C)
    l9, st9 = res.call(9, 0.5, 3.0)
    l10, st10 = res.call(10, 0.5, 3.0)
    again, st = res.call(10, 0.5, 3.0)
    assert st9 == st10 == st == 0
    assert np.array_equal(l9.view(np.uint32), l10.view(np.uint32))
    assert np.array_equal(l10.view(np.uint32), again.view(np.uint32))


# tile ids of hip_sgemm_tile_split with an assembly loop: 0 = 256 x 128,
# 1 = 128 x 128, 6 = 64 x 64 (64-deep stages, four K-slice wavefronts)
TILE_SHAPES = {0: (256, 128), 1: (128, 128), 6: (64, 64)}


@pytest.mark.parametrize("tile", sorted(TILE_SHAPES))
@pytest.mark.parametrize("gm,gn,K", [(1, 1, 16), (2, 3, 144), (3, 2, 1008), (1, 1, 40), (2, 2, 7),
                                     (2, 1, 33), (4, 4, 4097)])
def test_tile_api_whole_tiles(tile, gm, gn, K):
    """hip_sgemm_tile_split(tile, 1) takes the assembly loop on a grid of
    gm x gn whole tiles: one stage, odd and even stage counts, ragged first
    stages; and with one extra row, a partial bottom edge."""
    bm, bn = TILE_SHAPES[tile]
    for M, N in ((gm * bm, gn * bn), (gm * bm + 1, gn * bn)):
        print(f"[kloop tile api] tile {tile}: {M}x{N}x{K}", flush=True)
        A, B, C = inputs.make_abc(M, N, K, 12800 + M + K + tile)

        def call(*args):
            return sgemm.hip_sgemm_tile_split(tile, 1, *args)
        out, st = gh.run(gh.Case(M, N, K, 0.5, 3.0, A, B, C), call)
        assert st == 0
        ref = oracle.oracle_sgemm(A, B, C, 0.5, 3.0)
        assert oracle.normalised_error(out, ref, C, 0.5, 3.0, strict=True) <= BOUND


OPS = [("N", "N"), ("N", "T"), ("T", "N"), ("T", "T")]


@pytest.mark.parametrize("M,N,K", [(4096, 4096, 48), (4096, 4096, 1001), (2048, 2048, 300),
                                   (2048 + 7, 2048 + 9, 77)])
def test_kloop_every_orientation_bit_identical(M, N, K):
    """Every orientation of the operands runs the same loop on the same LDS
    contents (only the stage loads and stores differ), so all four give the
    same bits; they are checked against the reference as well."""
    print(f"[kloop orientations] {M}x{N}x{K}", flush=True)
    A, B, C = inputs.make_abc(M, N, K, 13200 + M + K)
    ref = oracle.oracle_sgemm(A, B, C, 0.5, 3.0)
    outs = {}
    for op_a, op_b in OPS:
        sa = np.ascontiguousarray(A.T) if op_a == "T" else A
        sb = np.ascontiguousarray(B.T) if op_b == "T" else B
        case = gh.Case(M, N, K, 0.5, 3.0, sa, sb, C, sa.shape[1] + 1, sb.shape[1] + 3, N + 2)

        def call(*args, op_a=op_a, op_b=op_b):
            return sgemm.hip_sgemm_ex(op_a, op_b, *args)
        out, st = gh.run(case, call)
        assert st == 0
        err = oracle.normalised_error(out, ref, C, 0.5, 3.0, strict=True)
        assert err <= BOUND, (op_a, op_b, err)
        outs[op_a + op_b] = out
    for key in ("NT", "TN", "TT"):
        assert np.array_equal(outs["NN"].view(np.uint32), outs[key].view(np.uint32)), key


@pytest.mark.parametrize("tile", sorted(TILE_SHAPES))
def test_tile_api_padded_misaligned_nan_c(tile):
    bm, bn = TILE_SHAPES[tile]
    M, N, K = 2 * bm, 3 * bn, 75
    print(f"[kloop tile api alignment] tile {tile}: {M}x{N}x{K}", flush=True)
    A, B, _ = inputs.make_abc(M, N, K, 12900 + tile)
    nanC = np.full((M, N), np.nan, np.float32)

    def call(*args):
        return sgemm.hip_sgemm_tile_split(tile, 1, *args)
    out, st = gh.run(gh.Case(M, N, K, -1.5, 0.0, A, B, nanC, K + 3, N + 5, N + 7, 1, 2, 3), call)
    assert st == 0 and np.all(np.isfinite(out))
    ref = oracle.oracle_sgemm(A, B, None, -1.5, 0.0)
    assert oracle.normalised_error(out, ref, None, -1.5, 0.0, strict=True) <= BOUND


@pytest.mark.parametrize("M,N,K", [(2048, 2048, 2048), (2048, 2048, 2053), (2048, 4096, 1024),
                                   (2048 + 3, 2048 + 11, 500)])
def test_dispatch_128_tiles(M, N, K):
    """Level 10 on 128 x 128 grids (one or more tiles per CU, plus fringes)
    takes the 128 x 128 assembly loop."""
    print(f"[kloop 128] {M}x{N}x{K}", flush=True)
    A, B, C = inputs.make_abc(M, N, K, 13000 + M + N + K)
    out, st = gh.run(gh.Case(M, N, K, 0.5, 3.0, A, B, C), 10)
    assert st == 0
    ref = oracle.oracle_sgemm(A, B, C, 0.5, 3.0)
    assert oracle.normalised_error(out, ref, C, 0.5, 3.0, strict=True) <= BOUND


def test_loops_deterministic_and_agree():
    """Every loop is deterministic; the 256 x 128 and 128 x 128 loops give
    each output the same chain of MFMAs over the same k (16-deep stages,
    k = 4 s + lane / 16 in MFMA step s), so their results agree bit for
    bit."""
    M = N = 2048
    K = 512
    A, B, C = inputs.make_abc(M, N, K, 13100)
    outs = []
    for tile in (0, 1, 6):
        def call(*args, tile=tile):
            return sgemm.hip_sgemm_tile_split(tile, 1, *args)
        a, st1 = gh.run(gh.Case(M, N, K, 0.5, 3.0, A, B, C), call)
        b, st2 = gh.run(gh.Case(M, N, K, 0.5, 3.0, A, B, C), call)
        assert st1 == st2 == 0
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), tile
        outs.append(a)
    # tiles 0 and 1 accumulate every output in the same order (16-deep
    # stages, k = 4 s + lane/16 per MFMA step, one chain per block); tile 6
    # adds four K slices' chains, another order
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))


@pytest.mark.parametrize("tile", sorted(TILE_SHAPES))
@pytest.mark.parametrize("splits", [2, 3, 7])
def test_kloop_split_k(tile, splits):
    """hip_sgemm_tile_split(tile, splits) on whole tiles runs the assembly
    loops over K slices (each slice's first stage takes its own K % 16
    leftover; the last slice is short) and the in-order reduction."""
    bm, bn = TILE_SHAPES[tile]
    M, N, K = 2 * bm, 3 * bn, 1001
    print(f"[kloop split] tile {tile} {M}x{N}x{K} in {splits}", flush=True)
    A, B, C = inputs.make_abc(M, N, K, 13300 + tile + splits)

    def call(*args):
        return sgemm.hip_sgemm_tile_split(tile, splits, *args)
    out, st = gh.run(gh.Case(M, N, K, 0.5, 3.0, A, B, C), call)
    assert st == 0
    ref = oracle.oracle_sgemm(A, B, C, 0.5, 3.0)
    assert oracle.normalised_error(out, ref, C, 0.5, 3.0, strict=True) <= BOUND


@pytest.mark.parametrize("tile", sorted(TILE_SHAPES))
def test_kloop_split_k_integer_exact_deterministic(tile):
    bm, bn = TILE_SHAPES[tile]
    M, N, K = 2 * bm, 2 * bn, 1500
    A, B, C = inputs.integer_abc(M, N, K, seed=13400 + tile)
    ref = oracle.oracle_sgemm(A, B, C, 2.0, -1.0)

    def call(*args):
        return sgemm.hip_sgemm_tile_split(tile, 6, *args)
    first, st = gh.run(gh.Case(M, N, K, 2.0, -1.0, A, B, C), call)
    again, st2 = gh.run(gh.Case(M, N, K, 2.0, -1.0, A, B, C), call)
    assert st == st2 == 0
    assert np.array_equal(first.astype(np.float64), ref.ref)
    assert np.array_equal(first.view(np.uint32), again.view(np.uint32))


@pytest.mark.parametrize("M,N,K", [(512, 512, 8192), (700, 600, 8200)])
def test_kloop_split_k_every_orientation(M, N, K):
    """Level 10's split-K plan (512 x 512 x 8192: 64 whole 64 x 64 tiles in
    8 slices; 700 x 600 x 8200: 110 tiles with partial bottom and right
    edges in 4 slices, ragged K) in every orientation through hip_sgemm_ex:
    the same bits, within the bound."""
    print(f"[kloop split orientations] {M}x{N}x{K}", flush=True)
    assert sgemm.hip_sgemm_plan(M, N, K)["name"] == "split_k"
    A, B, C = inputs.make_abc(M, N, K, 13500 + M)
    ref = oracle.oracle_sgemm(A, B, C, 1.0, 1.0)
    outs = {}
    for op_a, op_b in OPS:
        sa = np.ascontiguousarray(A.T) if op_a == "T" else A
        sb = np.ascontiguousarray(B.T) if op_b == "T" else B

        def call(*args, op_a=op_a, op_b=op_b):
            return sgemm.hip_sgemm_ex(op_a, op_b, *args)
        out, st = gh.run(gh.Case(M, N, K, 1.0, 1.0, sa, sb, C, sa.shape[1] + 1, sb.shape[1] + 3,
                                 N + 2), call)
        assert st == 0
        assert oracle.normalised_error(out, ref, C, 1.0, 1.0, strict=True) <= BOUND
        outs[op_a + op_b] = out
    for key in ("NT", "TN", "TT"):
        assert np.array_equal(outs["NN"].view(np.uint32), outs[key].view(np.uint32)), key


EDGE_SHAPES = [(1000, 700, 300), (3000, 3000, 77), (65, 4097, 129), (4097, 65, 33), (777, 1029, 1000),
               (2049, 2047, 16)]


@pytest.mark.parametrize("tile", sorted(TILE_SHAPES))
@pytest.mark.parametrize("M,N,K", EDGE_SHAPES)
def test_kloop_edge_tiles_every_orientation(tile, M, N, K):
    """Grids whose bottom and right tiles are partial: the loads past M / N
    read zeros or elements only out-of-range outputs use, the epilogue
    stores only inside the matrix (the harness's guard regions and padding
    check that), and every orientation gives the same bits."""
    print(f"[kloop edges] tile {tile} {M}x{N}x{K}", flush=True)
    A, B, C = inputs.make_abc(M, N, K, 13600 + M + N + K + tile)
    ref = oracle.oracle_sgemm(A, B, C, 0.5, 3.0)
    outs = {}
    for op_a, op_b in OPS:
        sa = np.ascontiguousarray(A.T) if op_a == "T" else A
        sb = np.ascontiguousarray(B.T) if op_b == "T" else B
        case = gh.Case(M, N, K, 0.5, 3.0, sa, sb, C, sa.shape[1] + 3, sb.shape[1] + 1, N + 5)

        def call(*args, op_a=op_a, op_b=op_b):
            if op_a == "N" and op_b == "N":
                return sgemm.hip_sgemm_tile_split(tile, 1, *args)
            return sgemm.hip_sgemm_ex(op_a, op_b, *args)
        out, st = gh.run(case, call)
        assert st == 0
        err = oracle.normalised_error(out, ref, C, 0.5, 3.0, strict=True)
        assert err <= BOUND, (op_a, op_b, err)
        outs[op_a + op_b] = out
    if tile == 6:
        # level 10 (hip_sgemm_ex) takes the same 64 x 64 loop on these grids
        for key in ("NT", "TN", "TT"):
            assert np.array_equal(outs["NN"].view(np.uint32), outs[key].view(np.uint32)), key


@pytest.mark.parametrize("tile", sorted(TILE_SHAPES))
def test_kloop_edge_tiles_nan_c_misaligned(tile):
    M, N, K = 1000, 700, 300
    A, B, _ = inputs.make_abc(M, N, K, 13700 + tile)
    nanC = np.full((M, N), np.nan, np.float32)

    def call(*args):
        return sgemm.hip_sgemm_tile_split(tile, 1, *args)
    out, st = gh.run(gh.Case(M, N, K, -1.5, 0.0, A, B, nanC, K + 3, N + 5, N + 7, 1, 2, 3), call)
    assert st == 0 and np.all(np.isfinite(out))
    ref = oracle.oracle_sgemm(A, B, None, -1.5, 0.0)
    assert oracle.normalised_error(out, ref, None, -1.5, 0.0, strict=True) <= BOUND


@pytest.mark.parametrize("tile", sorted(TILE_SHAPES))
def test_kloop_edge_tiles_integer_exact_and_split(tile):
    """Integer data on a partial grid, unsplit and in 3 K parts: exact."""
    M, N, K = 600, 520, 1300
    A, B, C = inputs.integer_abc(M, N, K, seed=13800 + tile)
    ref = oracle.oracle_sgemm(A, B, C, 1.0, -1.0)
    for splits in (1, 3):
        def call(*args, splits=splits):
            return sgemm.hip_sgemm_tile_split(tile, splits, *args)
        out, st = gh.run(gh.Case(M, N, K, 1.0, -1.0, A, B, C), call)
        assert st == 0
        assert np.array_equal(out.astype(np.float64), ref.ref), splits
