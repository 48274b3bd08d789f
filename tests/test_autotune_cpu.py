"""The tuning sweep's host side (no GPU): argument and shape parsing, the
slice arithmetic it shares with hip_sgemm_tile_split, and the committed
sweep table (profiles/autotune_sweep_all_tiles.md) against the dispatcher:
for every swept shape hip_sgemm must still take the plan and configuration
recorded there, and that configuration (or, for plans that are not a
single tile configuration, hip_sgemm itself) must be within the stated
tolerance of the fastest configuration measured."""

from __future__ import annotations

import os

import pytest

from dense_fp32_matrix_row_amd import autotune, sgemm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TABLE = os.path.join(ROOT, "profiles", "autotune_sweep_all_tiles.md")


def test_parse_shape():
    assert autotune.parse_shape("1024") == (1024, 1024, 1024)
    assert autotune.parse_shape(" 700x600X8200 ") == (700, 600, 8200)
    for bad in ("", "1x2", "0", "1x2x-3", "axbxc"):
        with pytest.raises(ValueError):
            autotune.parse_shape(bad)


def test_parse_args():
    a = autotune.parse_args(["--shapes", "256,2048x2048x8192", "--splits", "4,1,4", "--reps", "3"])
    assert a.shape_list == [(256, 256, 256), (2048, 2048, 8192)]
    assert a.split_list == [1, 4] and a.reps == 3
    d = autotune.parse_args([])
    assert len(d.shape_list) == len(autotune.DEFAULT_SHAPES)
    for bad in (["--splits", "0"], ["--reps", "0"], ["--shapes", ","]):
        with pytest.raises(SystemExit):
            autotune.parse_args(bad)


def test_tile_bk_and_slices():
    names = [sgemm.hip_sgemm_tile_name(t) for t in range(sgemm.hip_sgemm_num_tiles())]
    assert [autotune.tile_bk(n) for n in names[:7]] == [16, 32, 16, 16, 32, 32, 64]
    assert autotune.k_split_for(8200, 4, 64) == 2112 and autotune.slices(8200, 4, 64) == 4
    assert autotune.slices(1000, 1, 16) == 1 and autotune.slices(64, 16, 64) == 1
    # the split plan's workspace is slices x M x N floats: the same slice count
    for M, N, K in [(512, 512, 8192), (700, 600, 8200), (768, 768, 4096)]:
        plan, tile, s = autotune.dispatch_pick(sgemm, M, N, K)
        assert plan == "split_k" and tile == 6
        assert sgemm.hip_sgemm_plan(M, N, K)["workspace_bytes"] == s * M * N * 4


def test_table_round_trips():
    rows = [{"M": 2, "N": 3, "K": 4, "plan": "tiles", "pick": "0/1", "pick_tflops": 1.5,
             "auto_tflops": 1.25, "best": "0/1", "best_name": "x", "best_tflops": 1.5,
             "top": ["1/1=1.0"], "configs": 5}]
    back = autotune.read_table(autotune.render_table(rows, ["a"], None))
    assert back == [{"M": 2, "N": 3, "K": 4, "plan": "tiles", "pick": "0/1", "pick_tflops": 1.5,
                     "auto_tflops": 1.25, "best": "0/1", "best_tflops": 1.5}]


def _rows():
    with open(TABLE) as f:
        rows = autotune.read_table(f.read())
    assert len(rows) >= 15
    return rows


def test_dispatch_picks_are_the_swept_ones():
    """A change of the dispatch rules or their constants that moves any
    swept shape to another plan or configuration fails here until the sweep
    is re-run and the table re-committed."""
    for r in _rows():
        plan, tile, s = autotune.dispatch_pick(sgemm, r["M"], r["N"], r["K"])
        assert plan == r["plan"], (r["M"], r["N"], r["K"])
        assert (f"{tile}/{s}" if tile is not None else "-") == r["pick"], (r["M"], r["N"], r["K"])


def test_dispatch_picks_are_within_tolerance_of_the_fastest():
    """The pick's own measurement where it is one configuration (hip_sgemm
    runs the same kernels; its separately timed figure carries a few
    percent of launch-to-launch spread at these sizes), hip_sgemm's where
    the plan is not one configuration."""
    for r in _rows():
        floor = (1.0 - autotune.TOLERANCE) * r["best_tflops"]
        measured = r["pick_tflops"] if r["pick_tflops"] is not None else r["auto_tflops"]
        assert measured >= floor, r
