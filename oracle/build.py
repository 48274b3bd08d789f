"""Build the CPU reference library (liboracle_sgemm.so) with gcc.

Test infrastructure only; shares nothing with the HIP library's build.
"""

from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "oracle_sgemm.c")
LIBRARY = os.path.join(HERE, "liboracle_sgemm.so")

# -ffp-contract=off: no fused multiply-add may change the float64 rounding;
# -fno-fast-math: keep IEEE semantics (fabs, ordering of the sum).
CFLAGS = ["-O2", "-fPIC", "-shared", "-std=c11", "-ffp-contract=off",
          "-fno-fast-math", "-pthread", "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    tmp = LIBRARY + ".tmp"
    cmd = ["gcc", *CFLAGS, "-o", tmp, SOURCE, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose=True))
