"""Build libsgemm.so (the HIP kernels and the C-ABI host layer) for gfx950.

Each .hip source is compiled separately (in parallel) with hipcc and the
objects are linked into dense_fp32_matrix_row_amd/libsgemm.so, next to the
Python binding that loads it.  l10_kloop.hip is also compiled to assembly,
and the library is not linked unless its loop kernels pass the
staging-register check below.
"""

from __future__ import annotations

import glob
import os
import re
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
    "-Wall", f"-I{INCLUDE}",
]


def hipcc() -> str:
    return os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


# The assembly K loops of l10_kloop.hip are two asm statements per kernel: a
# prelude whose buffer loads are still in flight when it ends (they fill the
# staging registers, which the compiler sees only as the statement's
# outputs) and the loop, which consumes them.  Code the compiler places
# between the two must not touch those registers: a copy would read values
# that have not arrived.  The build compiles the file to assembly and
# refuses to link a library in which it does.
KLOOP_SOURCE = os.path.join(CSRC, "l10_kloop.hip")
FIRST_STAGING = 80
# last staging register per block tile (DEPTH sets of a stage's A and B
# float4s from v80, as gen_kloop.py lays them out); a fringe variant also
# stages one word of the extra row and one of the extra column per set,
# right after them
LAST_STAGING = {256: 80 + 12 - 1, 128: 80 + 2 * 16 - 1, 64: 80 + 2 * 32 - 1}
FRINGE_SETS = {256: 1, 128: 2, 64: 2}
# 3 tiles x 4 orientations x (plain, split K, fringe variant)
KLOOP_KERNELS = 36


def kloop_kernels(asm: str):
    """(name, instruction lines) of every loop kernel in the assembly."""
    starts = [m.start() for m in re.finditer(r"^_ZN5sgemm\S*k_kloop\S*:", asm, re.M)]
    for i, st in enumerate(starts):
        body = asm[st:starts[i + 1] if i + 1 < len(starts) else len(asm)]
        yield body.split(":", 1)[0], [ln.split(";")[0].strip() for ln in body.split("\n")]


def _registers(ins: str):
    regs = [(int(a), int(b)) for a, b in re.findall(r"\bv\[(\d+):(\d+)\]", ins)]
    return regs + [(int(r), int(r)) for r in re.findall(r"\bv(\d+)\b", ins)]


def check_kloop_staging(asm: str) -> list:
    """Violations (kernel, problem) of the staging-register rule; empty when
    every loop kernel is sound."""
    bad = []
    kernels = list(kloop_kernels(asm))
    if len(kernels) != KLOOP_KERNELS:
        bad.append(("*", f"{len(kernels)} loop kernels found, expected {KLOOP_KERNELS}"))
    for name, lines in kernels:
        # KTile<BM, BN, BK, KS, TA, TB, FR> as mangled
        m = re.search(r"KTileILi(\d+)ELi\d+ELi\d+ELi\d+ELb[01]ELb[01]ELb([01])E", name)
        bm = int(m.group(1)) if m else None
        last = LAST_STAGING.get(bm) if m else None
        if m and last is not None and m.group(2) == "1":
            last += 2 * FRINGE_SETS[bm]
        if last is None or "s_nop 4" not in lines:
            bad.append((name, "no prelude found"))
            continue
        start = lines.index("s_nop 4")               # the prelude's first line
        try:
            end = lines.index("s_barrier", start)    # the loop statement's barrier
        except ValueError:
            bad.append((name, "no loop barrier after the prelude"))
            continue
        prelude_words = 0  # staging registers the prelude's loads fill
        for ins in lines[start:end]:
            if not ins or ins.startswith((".", "s_")):
                continue
            lm = re.match(r"buffer_load_dword(x4)? v\[?(\d+)(:\d+\])?, \S+, \S+, \S+ offen$", ins)
            if lm and FIRST_STAGING <= int(lm.group(2)) <= last:
                prelude_words += 4 if lm.group(1) else 1
                continue
            if [r for r in _registers(ins) if r[1] >= FIRST_STAGING and r[0] <= last]:
                bad.append((name, f"touches a staging register before the loop: {ins}"))
        if prelude_words != last - FIRST_STAGING + 1:
            bad.append((name, f"prelude loads fill {prelude_words} staging registers of "
                              f"v{FIRST_STAGING}..v{last}"))
    return bad


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs, procs = [], []
    kloop_asm = os.path.join(BUILD_DIR, "l10_kloop.s")
    compiles = [[hipcc(), *HIPCC_FLAGS, "--cuda-device-only", "-S", KLOOP_SOURCE, "-o", kloop_asm]]
    for src in sources():
        obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
        compiles.append([hipcc(), *HIPCC_FLAGS, "-c", src, "-o", obj])
        objs.append(obj)
    for cmd in compiles:
        if verbose:
            print(" ".join(cmd), flush=True)
        src = cmd[-3]
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        if len(procs) >= jobs:
            _reap(procs.pop(0))
    for pr in procs:
        _reap(pr)
    with open(kloop_asm) as f:
        bad = check_kloop_staging(f.read())
    if bad:
        raise RuntimeError("l10_kloop.hip: compiled code breaks the staging-register rule; not linking:\n"
                           + "\n".join(f"  {k}: {why}" for k, why in bad))
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
