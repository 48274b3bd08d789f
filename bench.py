#!/usr/bin/env python3
"""Benchmark of libsgemm on one MI355X.

Default: the 4096^3 workload (alpha = 0.5, beta = 3, i.i.d. uniform[-1, 1]
inputs from seed 1003) through hip_sgemm (the library's own kernel choice),
W untimed warm-up calls (continued until at least 300 ms of back-to-back
calls, so the clocks have left their ramp from idle; the calls and
milliseconds spent are reported), then exactly K timed calls, each on its own freshly
filled copy of C (so every step computes C <- 0.5*A@B + 3*C from the same
pristine inputs, and no restore copy sits inside the timed region).  Inputs
are resident in HBM before timing starts.

Prints one JSON line: TFLOPS over the timed region (2*M*N*K per step, host
clock), the dominant kernel's roofline (its average duration per launch from
the two HIP events on the launch stream that bracket the timed region's K
back-to-back calls, against the 157.3 TFLOP/s FP32 matrix peak), and the
CPU reference timed on the host on a bounded sample of the same problem
(its first rows), whose output also checks the GPU's rows.  The timed
region holds no per-call events: an event pair around every call leaves
an idle gap between consecutive kernels (back to back there is none) and
costs the timed region about 1 % at 4096^3 (measured); the kernels
themselves run as long either way.  The
per-call median, mean and min come from a second pass of K calls after the
timed region, one event pair around each call, and are reported beside the
line's figures.

Options: --level L forces a ladder rung (hip_sgemm_level); --workload picks
another of the five problem sizes; --ladder PATH times every level on every
workload (median of the per-launch event times), the vendor BLAS beside them
and the CPU reference on each whole problem (all host cores; also one thread
for 256^3 and 1024^3), and writes one JSON line per record to PATH (the
headline line is still printed last); --no-cpu skips the CPU legs.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "SGEMM TFLOPS at M=N=K=4096 (fraction of FP32 peak) on one MI355X"
# MI355X FP32 peak, 256 CUs x 256 FLOP/clk x 2.4 GHz: the matrix-core rate of
# v_mfma_f32_32x32x2_f32, and also the vector rate of VOP2 v_fmac_f32 (the
# VOP3 v_fma_f32 form issues at half that rate).
PEAK_FP32_TFLOPS = 157.3
PROFILES = os.path.join(ROOT, "profiles")
# Every timed region is preceded by at least this much back-to-back work
# (and at least the requested warm-up calls): from idle, MI355X's clocks
# take ~30 calls of the 4096^3 problem (~30 ms) to reach steady state, and
# calls timed inside that ramp run up to 15 % slow.
WARM_MS = 300.0


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    # MI355X takes ~30 back-to-back 4096^3 calls (~35 ms) to ramp its clocks
    # up from idle; 50 warm-up calls reach the steady state.
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--warm-ms", type=float, default=WARM_MS,
                    help="minimum milliseconds of back-to-back warm-up calls before each timed "
                         "region (default %(default)s; 0 = exactly --warmup calls, as for "
                         "hardware-counter passes that serialise every dispatch)")
    ap.add_argument("--level", type=int, default=None)
    ap.add_argument("--workload", default="sgemm_4096")
    ap.add_argument("--ladder", default=None, metavar="PATH")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--vendor", action="store_true",
                    help="also time torch.addmm (the vendor BLAS) on the same workload, as context")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target CPU time of the reference sample")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run 10 device-to-device copies of MIB MiB (a kernel of "
                         "known traffic, to scale hardware byte counters) and exit")
    return ap.parse_args()


def _code_only(text: str) -> str:
    """C/C++ source without its comments and blank lines (string and
    character literals kept as written)."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return "\n".join(line.rstrip() for line in "".join(out).splitlines() if line.strip())


def kernel_source_digest() -> str:
    """Digest of the HIP sources without their comments, used to tell
    whether recorded hardware counters still describe the kernels being
    timed (an edit to a comment keeps it; any code change, host side
    included, makes a new one)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "dense_fp32_matrix_row_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".h", ".inc")):
            with open(os.path.join(csrc, name), encoding="utf-8") as f:
                h.update(name.encode() + b"\0" + _code_only(f.read()).encode())
    return h.hexdigest()[:16]


def recorded_traffic(workload: str, level_name: str):
    """HBM bytes per launch from committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    passes (profiles/pmc_traffic_<level>_<workload>.txt), or None when absent
    or taken on different kernel sources."""
    path = os.path.join(PROFILES, f"pmc_traffic_{level_name}_{workload}.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                fields[k.strip()] = v.strip()
    if fields.get("kernel_source_digest") != kernel_source_digest():
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


class Problem:
    def __init__(self, w, copies: int):
        import numpy as np
        import torch

        from dense_fp32_matrix_row_amd import inputs
        self.w = w
        A, B, C = inputs.make_workload(w)
        self.host = (A, B, C)
        self.dA = torch.from_numpy(A).cuda()
        self.dB = torch.from_numpy(B).cuda()
        self.dC0 = torch.from_numpy(C).cuda()
        self.copies = [torch.empty_like(self.dC0) for _ in range(copies)]
        del np

    def refill(self):
        for c in self.copies:
            c.copy_(self.dC0)


def warm_until(call, n: int, min_ms: float):
    """n calls, then more until at least min_ms of back-to-back calls (host
    clock, checked every 10 calls): the clocks ramp up from idle over tens
    of milliseconds, which a few calls of a short kernel do not cover.
    Returns (calls made, milliseconds spent)."""
    import torch
    t0 = time.perf_counter()
    i = 0
    while i < n or (min_ms > 0 and (time.perf_counter() - t0) * 1e3 < min_ms):
        call(i)
        i += 1
        if i % 10 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return i, (time.perf_counter() - t0) * 1e3


class Timing:
    """One timed region: host-clock ms per step over the whole region, and
    the per-launch kernel times from the HIP event pairs around each launch
    (mean, median, min), with the warm-up that preceded it."""

    def __init__(self, ms_per_step, kernel_ms_each, warm_calls, warm_ms):
        import statistics
        self.ms_per_step = ms_per_step
        self.kernel_ms_each = kernel_ms_each
        self.mean = sum(kernel_ms_each) / len(kernel_ms_each)
        self.median = statistics.median(kernel_ms_each)
        self.min = min(kernel_ms_each)
        self.warm_calls, self.warm_ms = warm_calls, warm_ms


def run_region(prob: Problem, level, steps: int, warmup: int, min_warm_ms: float = 0.0):
    """The headline's timed region: warm-up, then `steps` back-to-back calls
    on the current stream (the stream the library launches on) between two
    HIP events and two synchronisations.  Returns (host ms per step, event
    ms per call, warm-up calls, warm-up ms)."""
    import torch

    from dense_fp32_matrix_row_amd import sgemm
    w = prob.w
    stream = torch.cuda.current_stream()
    handle = stream.cuda_stream

    def call(c):
        args = (w.M, w.N, w.K, w.alpha, prob.dA, w.K, prob.dB, w.N, w.beta, c, w.N, handle)
        st = sgemm.hip_sgemm(*args) if level is None else sgemm.hip_sgemm_level(level, *args)
        if st != 0:
            raise RuntimeError(sgemm.hip_sgemm_status_string(st))

    prob.refill()
    torch.cuda.synchronize()
    warm_calls, warm_ms = warm_until(lambda i: call(prob.copies[i % len(prob.copies)]), warmup,
                                     min_warm_ms)
    prob.refill()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(steps):
        call(prob.copies[i])
    end.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    return (t1 - t0) * 1e3 / steps, start.elapsed_time(end) / steps, warm_calls, warm_ms


def run_timed(prob: Problem, level, steps: int, warmup: int, min_warm_ms: float = 0.0) -> Timing:
    """Warm-up and timed calls on the current stream (the stream the
    library launches on, so the events bracket its kernels), an event pair
    around each call."""
    import torch

    from dense_fp32_matrix_row_amd import sgemm
    w = prob.w
    stream = torch.cuda.current_stream()
    handle = stream.cuda_stream

    def call(c):
        args = (w.M, w.N, w.K, w.alpha, prob.dA, w.K, prob.dB, w.N, w.beta, c, w.N, handle)
        st = sgemm.hip_sgemm(*args) if level is None else sgemm.hip_sgemm_level(level, *args)
        if st != 0:
            raise RuntimeError(sgemm.hip_sgemm_status_string(st))

    prob.refill()
    torch.cuda.synchronize()
    warm_calls, warm_ms = warm_until(lambda i: call(prob.copies[i % len(prob.copies)]), warmup,
                                     min_warm_ms)
    prob.refill()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record(stream)
        call(prob.copies[i])
        ends[i].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    each = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    return Timing((t1 - t0) * 1e3 / steps, each, warm_calls, warm_ms)


def cpu_baseline(prob: Problem, gpu_out_rows, target_s: float):
    """The CPU reference on the first R rows of the same problem, R sized for
    about target_s seconds; returns the baseline record and the GPU's max
    normalised error on those rows."""
    import numpy as np

    from oracle import oracle
    A, B, C = prob.host
    w = prob.w
    probe = 32
    t = time.perf_counter()
    oracle.oracle_sgemm(np.ascontiguousarray(A[:probe]), B, np.ascontiguousarray(C[:probe]), w.alpha, w.beta)
    rate = probe / max(time.perf_counter() - t, 1e-6)          # rows per second
    rows = int(min(w.M, max(probe, (rate * target_s) // 32 * 32)))
    t = time.perf_counter()
    ref = oracle.oracle_sgemm(np.ascontiguousarray(A[:rows]), B, np.ascontiguousarray(C[:rows]),
                              w.alpha, w.beta)
    dt = time.perf_counter() - t
    out = gpu_out_rows(rows)
    err = oracle.normalised_error(out, ref, C[:rows], w.alpha, w.beta, strict=True)
    rec = {"value": 2.0 * rows * w.N * w.K / dt / 1e12, "unit": "TFLOPS", "cores": ref.threads,
           "kind": "oracle",
           "sample": f"rows 0..{rows - 1} of the {w.M}x{w.N}x{w.K} problem ({rows}x{w.N}x{w.K}, "
                     f"{dt:.1f} s, float64 accumulation)"}
    return rec, err


def device_info():
    import torch
    p = torch.cuda.get_device_properties(0)
    clock_mhz = None
    try:
        import ctypes
        # hipDeviceAttributeClockRate (kHz) through torch's HIP runtime
        lib = ctypes.CDLL("libamdhip64.so.7")
        val = ctypes.c_int()
        if lib.hipDeviceGetAttribute(ctypes.byref(val), 5, 0) == 0:   # hipDeviceAttributeClockRate
            clock_mhz = val.value / 1000.0
    except OSError:
        pass
    cus = p.multi_processor_count
    info = {"name": p.name, "gcn_arch": getattr(p, "gcnArchName", None), "cus": cus,
            "clock_mhz": clock_mhz}
    if clock_mhz:
        info["derived_fp32_peak_tflops"] = round(cus * 256 * clock_mhz * 1e6 / 1e12, 1)
    return info


def vendor_timed(prob: Problem, steps: int, warmup: int, min_warm_ms: float = 0.0) -> Timing:
    """The same call through torch.addmm on FP32 tensors (rocBLAS/hipBLASLt,
    TF32 off): a context figure for the vendor library, never a dependency of
    libsgemm.  Timed like run_timed (host clock not used)."""
    import torch
    torch.backends.cuda.matmul.allow_tf32 = False
    w = prob.w
    stream = torch.cuda.current_stream()
    prob.refill()
    torch.cuda.synchronize()
    wc, wms = warm_until(lambda i: prob.copies[i % len(prob.copies)].addmm_(
        prob.dA, prob.dB, beta=w.beta, alpha=w.alpha), warmup, min_warm_ms)
    prob.refill()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(ev):
        a.record(stream)
        prob.copies[i].addmm_(prob.dA, prob.dB, beta=w.beta, alpha=w.alpha)
        b.record(stream)
    torch.cuda.synchronize()
    return Timing(float("nan"), [a.elapsed_time(b) for a, b in ev], wc, wms)


def vendor_region(prob: Problem, steps: int) -> float:
    """The vendor call timed like the headline's region: `steps`
    back-to-back calls between two HIP events (run after vendor_timed, so
    the clocks are up).  Returns ms per call."""
    import torch
    w = prob.w
    stream = torch.cuda.current_stream()
    prob.refill()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(steps):
        prob.copies[i].addmm_(prob.dA, prob.dB, beta=w.beta, alpha=w.alpha)
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def bench_one(w, level, steps, warmup, prob=None, min_warm_ms=0.0):
    from dense_fp32_matrix_row_amd import sgemm
    prob = prob or Problem(w, max(steps, 1))
    timing = run_timed(prob, level, steps, warmup, min_warm_ms)
    eff_level = level if level is not None else sgemm.hip_sgemm_auto_level(
        w.M, w.N, w.K, prob.dA, w.K, prob.dB, w.N, prob.dC0, w.N)
    name = sgemm.hip_sgemm_level_name(eff_level)
    return prob, timing, eff_level, name


def ladder(args, steps: int, warmup: int) -> None:
    """Every level on every workload, the vendor BLAS beside them, and the
    CPU oracle on each whole problem: its wall clock (all host cores, and
    one thread for the two smallest workloads) and, against its result,
    every level's max normalised error over all of C (one more call on a
    fresh C after the timed ones)."""
    import torch

    from dense_fp32_matrix_row_amd import inputs, sgemm
    from oracle import oracle
    with open(args.ladder, "w") as f:
        def emit(rec, msg):
            f.write(json.dumps(rec) + "\n")
            f.flush()
            print(f"[ladder] {msg}", flush=True)

        for wl in inputs.WORKLOADS:
            prob = Problem(wl, max(steps, 1))
            A, B, C = prob.host
            ref = None
            if not args.no_cpu:
                for threads in ([0, 1] if wl.M <= 1024 else [0]):
                    t = time.perf_counter()
                    res = oracle.oracle_sgemm(A, B, C, wl.alpha, wl.beta, threads=threads)
                    dt = time.perf_counter() - t
                    ref = ref or res
                    emit({"workload": wl.name, "level": "oracle", "cores": res.threads,
                          "seconds": round(dt, 4), "gflops": round(wl.flops / dt / 1e9, 3),
                          "kind": "oracle (float64 accumulation, whole problem)"},
                         f"{wl.name} oracle on {res.threads} cores: {dt:.3f} s")
            for lv in range(sgemm.hip_sgemm_num_levels()):
                # the two naive rungs take 0.1-0.2 s per call at 4096: fewer calls
                slow = lv <= 1 and wl.M >= 2048
                st = min(steps, 3) if slow else min(steps, 20)
                wu = 1 if slow else min(warmup, 10)
                # short kernels: at least warm_ms of calls before timing
                _, tm, _, name = bench_one(wl, lv, st, wu, prob, 0.0 if slow else args.warm_ms)
                kms = tm.median
                tf = wl.flops / (kms * 1e-3) / 1e12
                rec = {"workload": wl.name, "level": lv, "level_name": name, "steps": st,
                       "warmup_calls": tm.warm_calls, "ms_per_step": round(tm.ms_per_step, 4),
                       "kernel_ms_median": round(tm.median, 4),
                       "kernel_ms_mean": round(tm.mean, 4), "kernel_ms_min": round(tm.min, 4),
                       "tflops": round(tf, 3), "frac_fp32_peak": round(tf / PEAK_FP32_TFLOPS, 4),
                       "algorithmic_gbs": round(wl.algorithmic_bytes / (kms * 1e-3) / 1e9, 1)}
                if ref is not None:
                    c = prob.copies[0]
                    c.copy_(prob.dC0)
                    sgemm.check(sgemm.hip_sgemm_level(lv, wl.M, wl.N, wl.K, wl.alpha, prob.dA, wl.K,
                                                      prob.dB, wl.N, wl.beta, c, wl.N, None))
                    torch.cuda.synchronize()
                    rec["max_normalised_error"] = oracle.normalised_error(
                        c.cpu().numpy(), ref, C, wl.alpha, wl.beta, strict=True)
                emit(rec, f"{wl.name} L{lv} {name}: median {kms:.4f} ms, {rec['tflops']} TFLOPS, "
                          f"error {rec.get('max_normalised_error')}")
            vt = vendor_timed(prob, min(steps, 20), min(warmup, 10), args.warm_ms)
            tf = wl.flops / (vt.median * 1e-3) / 1e12
            emit({"workload": wl.name, "level": "vendor",
                  "level_name": "torch.addmm (rocBLAS/hipBLASLt, FP32)",
                  "kernel_ms_median": round(vt.median, 4), "kernel_ms_mean": round(vt.mean, 4),
                  "kernel_ms_min": round(vt.min, 4), "tflops": round(tf, 3),
                  "frac_fp32_peak": round(tf / PEAK_FP32_TFLOPS, 4),
                  "algorithmic_gbs": round(wl.algorithmic_bytes / (vt.median * 1e-3) / 1e9, 1)},
                 f"{wl.name} vendor: median {vt.median:.4f} ms, {tf:.3f} TFLOPS")
            del prob, ref
            torch.cuda.empty_cache()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the kernel shards by C tiles across GPUs, but no multi-GPU path is built)",
              file=sys.stderr)
        return 2
    import torch

    from dense_fp32_matrix_row_amd import inputs, sgemm
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    torch.cuda.set_device(0)
    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.rand(n, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": 4 * n, "copy_calibration_bytes_written": 4 * n,
                          "copies": 10}), flush=True)
        return 0
    sgemm.load()
    w = inputs.WORKLOADS_BY_NAME[args.workload]
    steps, warmup = max(1, args.steps), max(0, args.warmup)

    if args.ladder:
        ladder(args, steps, warmup)

    prob = Problem(w, steps)
    ms, kms, warm_calls, warm_ms = run_region(prob, args.level, steps, warmup, args.warm_ms)
    # per-call times: a second pass of the same calls after the timed
    # region, one event pair around each (the clocks are still up)
    _, tm, lv, name = bench_one(w, args.level, steps, 0, prob=prob)
    tflops = w.flops / (ms * 1e-3) / 1e12
    achieved = w.flops / (kms * 1e-3) / 1e12
    # levels 9 and 10 run the matrix cores on every bench workload (level
    # 10's vector-ALU kernels only take problems with M or N <= 16)
    on_mfma = lv == 9 or (lv == 10 and min(w.M, w.N) > 16)
    roofline = {"bound": "mfma" if on_mfma else "alu", "achieved": round(achieved, 3),
                "peak": PEAK_FP32_TFLOPS,
                "unit": "TFLOP/s", "frac": None, "traffic": recorded_traffic(w.name, name)}
    roofline["frac"] = round(achieved / roofline["peak"], 4)
    line = {
        "metric": METRIC, "value": round(tflops, 3), "unit": "TFLOPS", "n_gpus": 1,
        "steps": steps, "warmup": warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp32",
        "data": "synthetic (i.i.d. uniform[-1,1], seeded)",
        "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K, "alpha": w.alpha,
                   "beta": w.beta, "level": lv, "level_name": name, "parallelism": "single GPU"},
        "roofline": roofline,
        "frac_fp32_peak": round(tflops / PEAK_FP32_TFLOPS, 4),
        "kernel_ms": round(kms, 4),
        "per_call_pass": {"kernel_ms_median": round(tm.median, 4), "kernel_ms_mean": round(tm.mean, 4),
                          "kernel_ms_min": round(tm.min, 4),
                          "tflops_at_median": round(w.flops / (tm.median * 1e-3) / 1e12, 3),
                          "note": "a second pass of the same calls after the timed region, "
                                  "one HIP event pair around each call"},
        "warmup_calls": warm_calls, "warmup_ms": round(warm_ms, 1),
        "algorithmic_gbs": round(w.algorithmic_bytes / (kms * 1e-3) / 1e9, 1),
        "device": device_info(),
    }
    if args.vendor:
        vt = vendor_timed(prob, steps, warmup, args.warm_ms)
        v_ms = vendor_region(prob, steps)
        line["vendor_blas"] = {"library": "torch.addmm (rocBLAS/hipBLASLt), FP32, TF32 off",
                               "kernel_ms": round(v_ms, 4),
                               "tflops": round(w.flops / (v_ms * 1e-3) / 1e12, 3),
                               "per_call_pass": {"kernel_ms_mean": round(vt.mean, 4),
                                                 "kernel_ms_median": round(vt.median, 4)},
                               "note": "context only; not part of libsgemm; kernel_ms between two "
                                       "HIP events around the back-to-back calls, as for kernel_ms "
                                       "above"}
    if not args.no_cpu:
        def rows_out(r):
            # one more call on a fresh C, outside any timed region
            c = prob.copies[0]
            c.copy_(prob.dC0)
            st = (sgemm.hip_sgemm if args.level is None else
                  (lambda *a: sgemm.hip_sgemm_level(args.level, *a)))(
                w.M, w.N, w.K, w.alpha, prob.dA, w.K, prob.dB, w.N, w.beta, c, w.N, None)
            if st != 0:
                raise RuntimeError(sgemm.hip_sgemm_status_string(st))
            torch.cuda.synchronize()
            return c[:r].cpu().numpy()
        rec, err = cpu_baseline(prob, rows_out, args.cpu_seconds)
        line["cpu_baseline"] = rec
        line["parity_max_normalised_error_on_sample"] = err
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
