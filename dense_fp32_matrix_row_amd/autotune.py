"""Sweep level 9's configurations (tile shape x K slices) per problem shape
through the C ABI and report the fastest, the way the pages tune block and
thread-tile sizes per GPU ([GEMM2], autotuning section: the best parameters
differ between GPUs, so they are searched, not derived).

Level 10's split-K choices come from this sweep on MI355X.  Run on a GPU:

    python -m dense_fp32_matrix_row_amd.autotune [--out sweep.jsonl] [--shapes 1024,2048x2048x8192]

Inputs are seeded uniform[-1, 1] matrices resident in device memory; each
configuration is timed with HIP events over `--reps` calls after `--warmup`
calls (the median is reported).  Every configuration computes the same
product, so correctness is the tests' business, not the sweep's.
"""

from __future__ import annotations

import argparse
import json
import sys

DEFAULT_SHAPES = ["256", "512", "768", "1024", "1536", "2048", "3072",
                  "1024x1024x4096", "1024x1024x8192", "2048x2048x8192", "512x512x8192",
                  "1024x4096x1024", "4096x1024x1024", "2048x4096x2048"]
DEFAULT_SPLITS = [1, 2, 3, 4, 6, 8, 12, 16]


def parse_shape(text: str):
    parts = [int(v) for v in text.lower().split("x")]
    return (parts * 3)[:3] if len(parts) == 1 else tuple(parts)


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--shapes", default=",".join(DEFAULT_SHAPES),
                    help="comma-separated MxNxK (or one size for a cube)")
    ap.add_argument("--splits", default=",".join(str(s) for s in DEFAULT_SPLITS))
    ap.add_argument("--reps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--out", default=None, help="also write one JSON record per line here")
    args = ap.parse_args(argv)

    import numpy as np
    import torch

    from dense_fp32_matrix_row_amd import sgemm

    if not torch.cuda.is_available():
        print("autotune needs a GPU", file=sys.stderr)
        return 2
    torch.cuda.set_device(0)
    sgemm.load()
    stream = torch.cuda.current_stream()
    splits_list = [int(s) for s in args.splits.split(",")]
    out = open(args.out, "w") if args.out else None
    ntiles = sgemm.hip_sgemm_num_tiles()

    # clocks ramp up over the first few dozen back-to-back calls after idle
    wab = torch.zeros(4096, 4096, device="cuda")
    wc = torch.empty(4096, 4096, device="cuda")
    for _ in range(40):
        sgemm.check(sgemm.hip_sgemm(4096, 4096, 4096, 1.0, wab, 4096, wab, 4096, 0.0, wc, 4096))
    torch.cuda.synchronize()
    del wab, wc

    for text in args.shapes.split(","):
        M, N, K = parse_shape(text)
        rng = np.random.default_rng(M * 31 + N * 7 + K)
        A = torch.from_numpy(rng.uniform(-1, 1, (M, K)).astype(np.float32)).cuda()
        B = torch.from_numpy(rng.uniform(-1, 1, (K, N)).astype(np.float32)).cuda()
        C = torch.empty(M, N, device="cuda")
        flops = 2.0 * M * N * K
        results = []
        # the host-side setup above leaves the GPU idle long enough for its
        # clocks to drop: run back to back for ~0.2 s before timing anything
        torch.cuda.synchronize()
        ramp = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ramp[0].record(stream)
        for i in range(1000):
            sgemm.check(sgemm.hip_sgemm(M, N, K, 1.0, A, K, B, N, 0.0, C, N, stream))
            if i % 10 == 9:
                ramp[1].record(stream)
                ramp[1].synchronize()
                if ramp[0].elapsed_time(ramp[1]) > 200.0:
                    break

        def timed(call):
            for _ in range(args.warmup):
                call()
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(args.reps)]
            for a, b in ev:
                a.record(stream)
                call()
                b.record(stream)
            torch.cuda.synchronize()
            return float(np.median([a.elapsed_time(b) for a, b in ev]))

        for tile in range(ntiles):
            for splits in splits_list:
                def call(tile=tile, splits=splits):
                    sgemm.check(sgemm.hip_sgemm_tile_split(tile, splits, M, N, K, 1.0, A, K, B, N,
                                                           0.0, C, N, stream))
                ms = timed(call)
                rec = {"M": M, "N": N, "K": K, "tile": tile, "tile_name": sgemm.hip_sgemm_tile_name(tile),
                       "splits": splits, "ms": round(ms, 5), "tflops": round(flops / (ms * 1e-3) / 1e12, 2)}
                results.append(rec)
                if out:
                    out.write(json.dumps(rec) + "\n")
        auto_ms = timed(lambda: sgemm.check(sgemm.hip_sgemm(M, N, K, 1.0, A, K, B, N, 0.0, C, N, stream)))
        best = max(results, key=lambda r: r["tflops"])
        print(f"{M}x{N}x{K}: best {best['tile_name']} splits {best['splits']} "
              f"{best['tflops']:.1f} TFLOP/s ({best['ms']:.4f} ms); hip_sgemm "
              f"{flops / (auto_ms * 1e-3) / 1e12:.1f} TFLOP/s; top 5: "
              + ", ".join(f"{r['tile_name']}/{r['splits']}={r['tflops']:.1f}"
                          for r in sorted(results, key=lambda r: -r["tflops"])[:5]), flush=True)
        del A, B, C
        torch.cuda.empty_cache()
    if out:
        out.close()
    return 0


if __name__ == "__main__":
    sys.exit(main())
