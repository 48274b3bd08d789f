"""bench.py end to end on the smallest workload: one JSON line with the
contract's fields (metric, value, unit, steps, warm-up, roofline with its
fraction, the per-call pass, the CPU reference's baseline and its parity
check on the GPU's rows), the timed region's figures consistent with each
other, and the benchmarked call within the error bound of the reference.
"""

from __future__ import annotations

import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_json_line_on_the_smallest_workload():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print("[bench] sgemm_256, 5 steps", flush=True)
    proc = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "sgemm_256",
                           "--steps", "5", "--warmup", "2", "--warm-ms", "0", "--cpu-seconds", "1"],
                          capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert proc.returncode == 0, proc.stderr[-2000:]
    lines = [ln for ln in proc.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1, proc.stdout
    rec = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline", "per_call_pass"):
        assert key in rec, key
    assert rec["n_gpus"] == 1 and rec["steps"] == 5 and rec["warmup"] == 2
    assert rec["config"]["workload"] == "sgemm_256"
    flops = 2 * 256 ** 3
    assert rec["value"] > 0 and abs(rec["value"] - flops / (rec["ms_per_step"] * 1e9)) < 1e-2 * rec["value"] + 1e-3
    roof = rec["roofline"]
    assert set(roof) >= {"bound", "achieved", "peak", "unit", "frac", "traffic"}
    assert roof["peak"] == 157.3 and 0 < roof["frac"] < 1
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    # the events lie inside the host-clock region
    assert rec["kernel_ms"] <= rec["ms_per_step"] * 1.001 + 2e-4
    base = rec["cpu_baseline"]
    assert base["kind"] == "oracle" and base["cores"] >= 1 and base["value"] > 0
    assert rec["parity_max_normalised_error_on_sample"] <= 1e-5
