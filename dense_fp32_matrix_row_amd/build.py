"""Build libsgemm.so (the HIP kernels and the C-ABI host layer) for gfx950.

Each .hip source is compiled separately (in parallel) with hipcc and the
objects are linked into dense_fp32_matrix_row_amd/libsgemm.so, next to the
Python binding that loads it.
"""

from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
REPO = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(REPO, "include")
BUILD_DIR = os.path.join(REPO, "_build", "libsgemm")
LIBRARY = os.path.join(HERE, "libsgemm.so")
ARCH = "gfx950"

# Packed FP32 instructions are switched off on purpose: the VALU rungs use
# plain v_fma_f32 (their roofline is the non-packed FP32 rate).
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-mcode-object-version=5",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", f"-I{INCLUDE}",
]


def hipcc() -> str:
    return os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs, procs = [], []
    for src in sources():
        obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
        cmd = [hipcc(), *HIPCC_FLAGS, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        objs.append(obj)
        if len(procs) >= jobs:
            _reap(procs.pop(0))
    for pr in procs:
        _reap(pr)
    tmp = LIBRARY + ".tmp"
    link = [hipcc(), f"--offload-arch={ARCH}", "-mcode-object-version=5", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.run(link, check=True)
    os.replace(tmp, LIBRARY)
    return LIBRARY


def _reap(item):
    src, proc = item
    out, _ = proc.communicate()
    if out.strip():
        sys.stderr.write(out)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed on {os.path.basename(src)} (exit {proc.returncode})")


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
