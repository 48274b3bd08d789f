"""Split K (hip_sgemm_tile_split) through the C ABI: every tile shape (the
seven named ones and the tile catalogue) with several slice counts on
whole, ragged-K and edge shapes against the CPU reference,
integer-valued data bit for bit, repeated calls bit-identical, beta = 0
never reading C, and nothing outside the C window written."""

from __future__ import annotations

import numpy as np
import pytest

from dense_fp32_matrix_row_amd import inputs, sgemm
from oracle import oracle
from tests import gpu_harness as gh

pytestmark = pytest.mark.gpu

BOUND = 1e-5
TILES = range(17)   # hip_sgemm_num_tiles(): 7 named tiles + a catalogue of 10


@pytest.fixture(scope="session", autouse=True)
def _device():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    sgemm.load()


def run_split(case: gh.Case, tile: int, splits: int):
    """gh.run (same guards) with hip_sgemm_tile_split as the call."""
    return gh.run(case, lambda *args: sgemm.hip_sgemm_tile_split(tile, splits, *args))


# whole tiles for every tile shape; whole M / N with a ragged K; edge tiles
SHAPES = [(256, 256, 1024), (512, 256, 1000), (300, 260, 1000), (129, 65, 777), (1024, 1024, 1024)]


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_split_matches_reference(tile, M, N, K):
    print(f"[split-K] tile {tile} {M}x{N}x{K}", flush=True)
    A, B, C = inputs.make_abc(M, N, K, 6000 + M + K + tile)
    ref = oracle.oracle_sgemm(A, B, C, 0.5, 3.0)
    for splits in (1, 2, 3, 5, 8, 64):
        out, st = run_split(gh.Case(M, N, K, 0.5, 3.0, A, B, C), tile, splits)
        assert st == 0, sgemm.hip_sgemm_status_string(st)
        err = oracle.normalised_error(out, ref, C, 0.5, 3.0, strict=True)
        assert err <= BOUND, (tile, splits, err)


@pytest.mark.parametrize("tile", TILES)
def test_split_padded_misaligned_beta0_nan(tile):
    """Padded strides, 4-byte-aligned bases, beta = 0 with C full of NaN
    (C must not be read): finite output within the bound."""
    M, N, K = 131, 257, 515
    A, B, _ = inputs.make_abc(M, N, K, 6100 + tile)
    nanC = np.full((M, N), np.nan, np.float32)
    case = gh.Case(M, N, K, 1.0, 0.0, A, B, nanC, K + 3, N + 5, N + 7, 1, 2, 3)
    out, st = run_split(case, tile, 4)
    assert st == 0 and np.all(np.isfinite(out))
    ref = oracle.oracle_sgemm(A, B, None, 1.0, 0.0)
    assert oracle.normalised_error(out, ref, None, 1.0, 0.0, strict=True) <= BOUND


@pytest.mark.parametrize("tile", TILES)
def test_split_integer_exact_and_deterministic(tile):
    """Integer entries in [-8, 8]: every partial sum (within a slice and
    across slices) is an integer far below 2^24, so the result is exact; two
    calls give the same bits."""
    M, N, K = 520, 390, 1500
    A, B, C = inputs.integer_abc(M, N, K, seed=6200 + tile)
    ref = oracle.oracle_sgemm(A, B, C, 2.0, -1.0)
    first = None
    for _ in range(2):
        out, st = run_split(gh.Case(M, N, K, 2.0, -1.0, A, B, C), tile, 6)
        assert st == 0
        assert np.array_equal(out.astype(np.float64), ref.ref)
        if first is None:
            first = out
        else:
            assert np.array_equal(first.view(np.uint32), out.view(np.uint32))


def test_split_random_data_deterministic():
    M, N, K = 1024, 1024, 4096
    A, B, C = inputs.make_abc(M, N, K, 6300)
    print("[split-K determinism] 1024x1024x4096, 128x128 tile, 8 slices", flush=True)
    a, st1 = run_split(gh.Case(M, N, K, 1.0, 1.0, A, B, C), 1, 8)
    b, st2 = run_split(gh.Case(M, N, K, 1.0, 1.0, A, B, C), 1, 8)
    assert st1 == st2 == 0
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_split_k_on_two_streams_at_once():
    """hip_sgemm's split-K plan on two streams with no synchronisation
    between them: each call takes its workspace from the pool in its own
    stream's order, so interleaved calls never share one.  Every result
    equals the same call made alone, bit for bit."""
    import torch
    M, N, K = 512, 512, 8192
    assert sgemm.hip_sgemm_plan(M, N, K)["name"] == "split_k"
    print("[split-K two streams] 512x512x8192, 6 calls per stream", flush=True)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    data = []
    for i in range(2):
        A, B, C = inputs.make_abc(M, N, K, 6400 + i)
        data.append(tuple(torch.from_numpy(x).cuda() for x in (A, B, C)))
    torch.cuda.synchronize()

    def call(i, out, stream):
        dA, dB, _ = data[i]
        st = sgemm.hip_sgemm(M, N, K, 1.5, dA, K, dB, N, -0.5, out, N, stream)
        assert st == 0, sgemm.hip_sgemm_status_string(st)

    alone = []
    for i in range(2):
        out = data[i][2].clone()
        torch.cuda.synchronize()
        call(i, out, streams[i])
        torch.cuda.synchronize()
        alone.append(out.cpu().numpy())
    outs = [[data[i][2].clone() for _ in range(6)] for i in range(2)]
    torch.cuda.synchronize()
    for r in range(6):
        for i in range(2):
            call(i, outs[i][r], streams[i])
    torch.cuda.synchronize()
    for i in range(2):
        for r in range(6):
            assert np.array_equal(outs[i][r].cpu().numpy().view(np.uint32), alone[i].view(np.uint32)), (i, r)
