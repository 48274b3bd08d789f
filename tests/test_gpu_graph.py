"""hip_sgemm inside a captured HIP graph (torch.cuda.graph records the
launches made on its capture stream, which the binding's default stream
argument resolves to).  One shape per plan of level 10's dispatcher: the
assembly-loop tiles, the tiles with a one-row / one-column fringe, split K
(its workspace is a stream-ordered pool allocation, captured as a graph
memory node), the thin kernels on the vector ALUs and on the matrix cores,
and the compiled small tiles.  Every replay must reproduce the eager call
bit for bit, with eager work and synchronisations between the replays, and
sampled rows must match the CPU reference."""

from __future__ import annotations

import numpy as np
import pytest

from dense_fp32_matrix_row_amd import inputs, sgemm
from oracle import oracle

pytestmark = pytest.mark.gpu

BOUND = 1e-5
REPLAYS = 3

# (M, N, K, alpha, beta)
SHAPES = [
    (2048, 2048, 512, 0.5, 3.0),    # assembly-loop tiles
    (4097, 4097, 64, 1.0, 1.0),     # 256x128 tiles whose blocks also sum one row and one column
    (2049, 2049, 64, 0.5, 3.0),     # the same beside 128x128 tiles
    (1025, 1025, 300, 1.0, 0.0),    # the same beside 64x64 tiles
    (4096 + 3, 4096 + 16, 64, 1.0, 1.0),  # tiles plus thin kernels on a 3-row / 16-column fringe
    (512, 512, 8192, 1.0, 0.0),     # split K
    (1, 4097, 1000, 1.0, 1.0),      # few rows, vector ALUs
    (3000, 3, 700, 2.0, -1.0),      # few columns, vector ALUs
    (16, 8192, 512, 1.0, 0.5),      # thin, matrix cores
    (300, 500, 100, 1.0, 0.0),      # small: thin kernel over 16-row panels
]


@pytest.fixture(scope="module", autouse=True)
def _device():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    sgemm.load()


@pytest.mark.parametrize("M,N,K,alpha,beta", SHAPES)
def test_graph_replays_match_eager(M, N, K, alpha, beta):
    import torch
    print(f"[graph] {M}x{N}x{K} alpha={alpha} beta={beta}", flush=True)
    A, B, C = inputs.make_abc(M, N, K, 4000 + M + N + K)
    dA, dB, dC0 = (torch.from_numpy(x).cuda() for x in (A, B, C))

    eager = dC0.clone()
    sgemm.check(sgemm.hip_sgemm(M, N, K, alpha, dA, K, dB, N, beta, eager, N))
    torch.cuda.synchronize()

    out = dC0.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        status = sgemm.hip_sgemm(M, N, K, alpha, dA, K, dB, N, beta, out, N)
    assert status == 0, sgemm.hip_sgemm_status_string(status)

    other = torch.ones(1 << 20, device="cuda")
    for rep in range(REPLAYS):
        out.copy_(dC0)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), eager.view(torch.int32)), f"replay {rep}"
        other.mul_(1.5).add_(out[0, 0])  # eager work between replays
        torch.cuda.synchronize()

    rows = np.unique(np.clip(np.array([0, 1, M // 2, M - 1]), 0, M - 1))
    ref = oracle.oracle_sgemm(np.ascontiguousarray(A[rows]), B, np.ascontiguousarray(C[rows]),
                              alpha, beta)
    got = out[torch.as_tensor(rows, device="cuda")].cpu().numpy()
    assert oracle.normalised_error(got, ref, C[rows], alpha, beta) <= BOUND


@pytest.mark.parametrize("M,N,K,alpha,beta", [(512, 512, 8192, 1.0, 0.0), (700, 600, 8200, 0.5, 2.0),
                                               (2048, 2048, 512, 0.5, 3.0)])
def test_noalloc_graph_replays_match_eager(M, N, K, alpha, beta):
    """hip_sgemm_ex_noalloc captured into a graph (the callers it is for):
    split K's partial sums then live in the library's fixed device array,
    so the graph holds no memory node; every replay equals the eager call
    (and hip_sgemm_ex) bit for bit, with eager work between replays."""
    import torch
    print(f"[graph no-alloc] {M}x{N}x{K} alpha={alpha} beta={beta}", flush=True)
    A, B, C = inputs.make_abc(M, N, K, 4100 + M + N + K)
    dA, dB, dC0 = (torch.from_numpy(x).cuda() for x in (A, B, C))

    eager = dC0.clone()   # the first call also looks the array's address up, outside the capture
    sgemm.check(sgemm.hip_sgemm_ex_noalloc("N", "N", M, N, K, alpha, dA, K, dB, N, beta, eager, N))
    pooled = dC0.clone()
    sgemm.check(sgemm.hip_sgemm_ex("N", "N", M, N, K, alpha, dA, K, dB, N, beta, pooled, N))
    torch.cuda.synchronize()
    assert torch.equal(eager.view(torch.int32), pooled.view(torch.int32))

    out = dC0.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        status = sgemm.hip_sgemm_ex_noalloc("N", "N", M, N, K, alpha, dA, K, dB, N, beta, out, N)
    assert status == 0, sgemm.hip_sgemm_status_string(status)

    other = torch.ones(1 << 20, device="cuda")
    for rep in range(REPLAYS):
        out.copy_(dC0)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), eager.view(torch.int32)), f"replay {rep}"
        other.mul_(1.5).add_(out[0, 0])
        torch.cuda.synchronize()
