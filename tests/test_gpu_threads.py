"""Calls from several host threads at once, each on a stream of its own:
the library keeps one workspace pool and one fixed workspace array per
device behind locks, and every call must still give the bits the same call
gives alone (run alone in a fresh process, the threads are also the pool's
first users, so its creation happens under contention).  Split K, which
takes its workspace from the pool (the fixed array of
hip_sgemm_ex_noalloc is shared by overlapping calls, so it is not used
here), and plans without workspace are mixed; every result is compared bit
for bit with a single-threaded call on the same inputs.
"""

from __future__ import annotations

import threading

import numpy as np
import pytest

from dense_fp32_matrix_row_amd import inputs, sgemm

pytestmark = pytest.mark.gpu

SHAPES = [(512, 512, 8192), (700, 600, 8200), (1024, 1024, 1024), (300, 260, 500), (5, 3001, 503)]
THREADS = 4
REPEATS = 3


@pytest.fixture(scope="module", autouse=True)
def _device():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    sgemm.load()


def test_threads_on_their_own_streams():
    import torch
    print(f"[threads] {THREADS} host threads x {REPEATS} rounds over {len(SHAPES)} shapes", flush=True)
    data = []
    for i, (M, N, K) in enumerate(SHAPES):
        A, B, C = inputs.make_abc(M, N, K, 32000 + i)
        data.append(tuple(torch.from_numpy(x).cuda() for x in (A, B, C)))
    assert any(sgemm.hip_sgemm_plan(*s)["name"] == "split_k" for s in SHAPES)

    errors = []
    got = {}

    def worker(t):
        try:
            torch.cuda.set_device(0)
            side = torch.cuda.Stream()
            with torch.cuda.stream(side):
                for rep in range(REPEATS):
                    # each thread walks the shapes in its own order
                    for j in range(len(SHAPES)):
                        i = (j + t) % len(SHAPES)
                        (M, N, K), (dA, dB, dC) = SHAPES[i], data[i]
                        c = dC.clone()
                        st = sgemm.hip_sgemm(M, N, K, 0.75, dA, K, dB, N, -1.5, c, N,
                                             side.cuda_stream)
                        if st != 0:
                            errors.append((t, i, sgemm.hip_sgemm_status_string(st)))
                            return
                        side.synchronize()
                        got[(t, rep, i)] = c.cpu().numpy()
        except Exception as e:  # reported by the main thread
            errors.append((t, repr(e)))

    torch.cuda.synchronize()
    threads = [threading.Thread(target=worker, args=(t,)) for t in range(THREADS)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
        assert not th.is_alive(), "a worker thread did not finish"
    assert not errors, errors
    assert len(got) == THREADS * REPEATS * len(SHAPES)
    # single-threaded results on the current stream, taken afterwards so
    # that in a fresh process the threads are the pool's first users
    want = []
    for (M, N, K), (dA, dB, dC) in zip(SHAPES, data):
        c = dC.clone()
        st = sgemm.hip_sgemm(M, N, K, 0.75, dA, K, dB, N, -1.5, c, N)
        assert st == 0, sgemm.hip_sgemm_status_string(st)
        torch.cuda.synchronize()
        want.append(c.cpu().numpy())
    for (t, rep, i), out in got.items():
        assert np.array_equal(out.view(np.uint32), want[i].view(np.uint32)), (t, rep, SHAPES[i])
