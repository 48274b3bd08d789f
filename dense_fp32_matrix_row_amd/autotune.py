"""Sweep every tile configuration x K-slice count per problem shape through
the C ABI, the way the pages tune a kernel's template parameters per GPU
([GEMM2], autotuning section: block tile, stage depth and per-thread tile
searched over their legal combinations, because the best set differs between
GPUs), and compare the fastest with what hip_sgemm's dispatcher picks.

The configurations are hip_sgemm_tile_split's tiles -- the seven named ones
(three of them level 10's assembly-loop tiles) and the catalogue of further
legal configurations of level 9's tile template (block tile, stage depth,
wavefront grid, matrix block size, K slices) -- each unsplit and over K
slices.  Run on a GPU:

    python -m dense_fp32_matrix_row_amd.autotune [--shapes 1024,2048x2048x8192]
        [--out sweep.jsonl] [--table sweep.md]

Inputs are seeded uniform[-1, 1] matrices resident in device memory; each
configuration is timed with HIP events over --reps calls after --warmup
calls (the median is kept), after at least 200 ms of back-to-back calls per
shape so that the clocks have ramped up.  Every configuration computes the
same product; correctness is the tests' business, not the sweep's.

--table writes one markdown row per shape: the dispatcher's plan and pick,
its time and hip_sgemm's, and the fastest configurations; the tests check
that the dispatcher still makes the picks recorded there and that each is
within the stated tolerance of the fastest.
"""

from __future__ import annotations

import argparse
import json
import sys

DEFAULT_SHAPES = ["256", "512", "768", "1024", "1536", "2048", "3072", "4096", "4097",
                  "1024x1024x4096", "1024x1024x8192", "2048x2048x8192", "512x512x8192",
                  "700x600x8200", "1024x4096x1024", "4096x1024x1024", "2048x4096x2048",
                  "5000x3000x2000", "300x300x3000", "2051x2055x300", "64x4096x4096", "4096x64x4096",
                  "128x4096x4096", "64x4096x1024", "32x4096x4096"]
DEFAULT_SPLITS = [1, 2, 3, 4, 6, 8, 12, 16]
# A pick counts as tuned when its time is within this fraction of the
# fastest configuration's on the same shape (box-to-box spread of these
# timings is about 1.5 %).
TOLERANCE = 0.05


def parse_shape(text: str):
    """'1024' -> (1024, 1024, 1024); '1024x512x77' -> (1024, 512, 77)."""
    parts = [int(v) for v in text.lower().strip().split("x")]
    if len(parts) not in (1, 3) or any(v <= 0 for v in parts):
        raise ValueError(f"shape must be N or MxNxK with positive sizes, got {text!r}")
    return tuple(parts * 3) if len(parts) == 1 else tuple(parts)


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--shapes", default=",".join(DEFAULT_SHAPES),
                    help="comma-separated MxNxK (or one size for a cube)")
    ap.add_argument("--splits", default=",".join(str(s) for s in DEFAULT_SPLITS))
    ap.add_argument("--reps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--out", default=None, help="one JSON record per configuration and shape")
    ap.add_argument("--table", default=None, help="markdown summary, one row per shape")
    args = ap.parse_args(argv)
    args.shape_list = [parse_shape(t) for t in args.shapes.split(",") if t.strip()]
    args.split_list = sorted({int(s) for s in args.splits.split(",") if s.strip()})
    if not args.shape_list or not args.split_list or min(args.split_list) < 1:
        ap.error("need at least one shape and split counts >= 1")
    if args.reps < 1 or args.warmup < 0:
        ap.error("--reps must be >= 1 and --warmup >= 0")
    return args


def tile_bk(name: str) -> int:
    """Stage depth BK of a tile from its name (block tile x BK first)."""
    return int(name.removeprefix("cat_").split("_")[0].split("x")[2])


def k_split_for(K: int, splits: int, bk: int) -> int:
    """The slice length hip_sgemm_tile_split uses: ceil(K / splits) rounded
    up to the tile's BK."""
    per = -(-K // splits)
    return -(-per // bk) * bk


def slices(K: int, splits: int, bk: int) -> int:
    """How many K slices a (tile, splits) request runs."""
    ks = k_split_for(K, splits, bk)
    return 1 if ks >= K else -(-K // ks)


def dispatch_pick(sgemm, M: int, N: int, K: int):
    """hip_sgemm's choice for a shape as (plan name, tile id, slices), with
    tile id and slices None for plans that are not a single
    hip_sgemm_tile_split configuration (thin kernels, fringes, panels)."""
    plan = sgemm.hip_sgemm_plan(M, N, K)["name"]
    g = sgemm.hip_sgemm_launch_shape(10, M, N, K)
    loop_tiles = {(256, 128): 0, (128, 128): 1, (64, 64): 6}
    if plan == "tiles":
        return plan, loop_tiles[(g["tile_m"], g["tile_n"])], 1
    if plan == "split_k":
        tiles = -(-M // 64) * -(-N // 64)
        return plan, 6, g["workgroups"] // tiles
    return plan, None, None


def main(argv=None) -> int:
    args = parse_args(argv)

    import numpy as np
    import torch

    from dense_fp32_matrix_row_amd import sgemm

    if not torch.cuda.is_available():
        print("autotune needs a GPU", file=sys.stderr)
        return 2
    torch.cuda.set_device(0)
    sgemm.load()
    stream = torch.cuda.current_stream()
    out = open(args.out, "w") if args.out else None
    rows = []
    ntiles = sgemm.hip_sgemm_num_tiles()
    names = [sgemm.hip_sgemm_tile_name(t) for t in range(ntiles)]

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

    for M, N, K in args.shape_list:
        rng = np.random.default_rng(M * 31 + N * 7 + K)
        A = torch.from_numpy(rng.uniform(-1, 1, (M, K)).astype(np.float32)).cuda()
        B = torch.from_numpy(rng.uniform(-1, 1, (K, N)).astype(np.float32)).cuda()
        C = torch.empty(M, N, device="cuda")
        flops = 2.0 * M * N * K

        def auto():
            sgemm.check(sgemm.hip_sgemm(M, N, K, 1.0, A, K, B, N, 0.0, C, N, stream))

        # the host-side setup leaves the GPU idle long enough for its clocks
        # to drop: run back to back for >= 200 ms before timing anything
        torch.cuda.synchronize()
        ramp = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ramp[0].record(stream)
        for i in range(100000):
            auto()
            if i % 10 == 9:
                ramp[1].record(stream)
                ramp[1].synchronize()
                if ramp[0].elapsed_time(ramp[1]) > 200.0:
                    break

        plan, pick_tile, pick_slices = dispatch_pick(sgemm, M, N, K)
        results = {}
        for tile in range(ntiles):
            bk = tile_bk(names[tile])
            wanted = list(args.split_list)
            if tile == pick_tile and pick_slices not in [slices(K, s, bk) for s in wanted]:
                wanted.append(pick_slices)
            for splits in wanted:
                s_count = slices(K, splits, bk)
                if (tile, s_count) in results:
                    continue

                def call(tile=tile, splits=splits):
                    sgemm.check(sgemm.hip_sgemm_tile_split(tile, splits, M, N, K, 1.0, A, K, B, N,
                                                           0.0, C, N, stream))
                ms = timed(call)
                rec = {"M": M, "N": N, "K": K, "tile": tile, "tile_name": names[tile],
                       "splits": splits, "slices": s_count, "ms": round(ms, 5),
                       "tflops": round(flops / (ms * 1e-3) / 1e12, 2)}
                results[(tile, s_count)] = rec
                if out:
                    out.write(json.dumps(rec) + "\n")
        auto_ms = timed(auto)
        ranked = sorted(results.values(), key=lambda r: r["ms"])
        best = ranked[0]
        pick = results.get((pick_tile, pick_slices)) if pick_tile is not None else None
        row = {"M": M, "N": N, "K": K, "plan": plan,
               "pick": f"{pick_tile}/{pick_slices}" if pick else "-",
               "pick_tflops": pick["tflops"] if pick else None,
               "auto_tflops": round(flops / (auto_ms * 1e-3) / 1e12, 2),
               "best": f"{best['tile']}/{best['slices']}", "best_name": best["tile_name"],
               "best_tflops": best["tflops"],
               "top": [f"{r['tile']}/{r['slices']}={r['tflops']}" for r in ranked[1:4]],
               "configs": len(results)}
        rows.append(row)
        if out:
            out.write(json.dumps({"summary": row}) + "\n")
            out.flush()
        print(f"{M}x{N}x{K}: plan {plan} pick {row['pick']} ({row['pick_tflops']}), hip_sgemm "
              f"{row['auto_tflops']} TFLOP/s; best {row['best']} {best['tile_name']} "
              f"{best['tflops']} over {len(results)} configurations", flush=True)
        del A, B, C
        torch.cuda.empty_cache()
    if out:
        out.close()
    if args.table:
        with open(args.table, "w") as f:
            f.write(render_table(rows, names, argv))
    return 0


TABLE_HEAD = ("| M | N | K | plan | pick (tile/slices) | pick TFLOP/s | hip_sgemm TFLOP/s | "
              "best (tile/slices) | best TFLOP/s | hip_sgemm / best | next fastest | configurations |")


def render_table(rows, names, argv) -> str:
    lines = ["| tile | name |", "|---|---|"]
    lines += [f"| {i} | {n} |" for i, n in enumerate(names)]
    lines += ["", TABLE_HEAD, "|" + "---|" * 12]
    for r in rows:
        lines.append(f"| {r['M']} | {r['N']} | {r['K']} | {r['plan']} | {r['pick']} | "
                     f"{r['pick_tflops'] if r['pick_tflops'] is not None else '-'} | {r['auto_tflops']} | "
                     f"{r['best']} | {r['best_tflops']} | {r['auto_tflops'] / r['best_tflops']:.3f} | "
                     f"{', '.join(r['top'])} | {r['configs']} |")
    return "\n".join(lines) + "\n"


def read_table(text: str):
    """Rows of a table written by render_table: dicts keyed like its header
    (M, N, K as ints; TFLOP/s as floats; '-' as None)."""
    keys = ["M", "N", "K", "plan", "pick", "pick_tflops", "auto_tflops", "best", "best_tflops"]
    out = []
    for line in text.splitlines():
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) != 12 or not cells[0].isdigit():
            continue
        rec = dict(zip(keys, cells[:9]))
        for k in ("M", "N", "K"):
            rec[k] = int(rec[k])
        for k in ("pick_tflops", "auto_tflops", "best_tflops"):
            rec[k] = None if rec[k] == "-" else float(rec[k])
        out.append(rec)
    return out


if __name__ == "__main__":
    sys.exit(main())
