"""Host-side check of the compiled assembly loops (no GPU): l10_kloop.hip is
compiled for gfx950 to assembly, and in every loop kernel the code the
compiler places between the prelude statement (stages 1 .. DEPTH requested
into the staging registers) and the loop statement (which consumes them)
must leave those registers alone.  Their loads are still in flight there
and the compiler does not know it: a copy of a staging register in that
stretch would read a value that has not arrived.
"""

from __future__ import annotations

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "dense_fp32_matrix_row_amd", "csrc")
HIPCC = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")

# last staging register per block tile (v80 onwards: DEPTH sets of the
# stage's A and B float4s), as gen_kloop.py lays them out
LAST_STAGING = {256: 80 + 12 - 1, 128: 80 + 2 * 16 - 1, 64: 80 + 2 * 32 - 1}


@pytest.fixture(scope="module")
def assembly(tmp_path_factory):
    if not os.path.exists(HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("isa") / "l10_kloop.s"
    cmd = [HIPCC if os.path.exists(HIPCC) else "hipcc", "--offload-arch=gfx950", "-O3",
           "-std=c++17", "-mcode-object-version=5", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", f"-I{os.path.join(ROOT, 'include')}", "--cuda-device-only", "-S",
           os.path.join(CSRC, "l10_kloop.hip"), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True, timeout=600)
    return out.read_text()


def _kernels(text):
    starts = [m.start() for m in re.finditer(r"^_ZN5sgemm\S*k_kloop\S*:", text, re.M)]
    for i, s in enumerate(starts):
        body = text[s:starts[i + 1] if i + 1 < len(starts) else len(text)]
        yield body.split(":", 1)[0], [l.split(";")[0].strip() for l in body.split("\n")]


def _registers(ins):
    regs = [(int(a), int(b)) for a, b in re.findall(r"\bv\[(\d+):(\d+)\]", ins)]
    return regs + [(int(r), int(r)) for r in re.findall(r"\bv(\d+)\b", ins)]


def test_staging_registers_untouched_between_prelude_and_loop(assembly):
    kernels = list(_kernels(assembly))
    assert len(kernels) == 24  # 3 tiles x 4 orientations x (plain, split K)
    for name, lines in kernels:
        last = LAST_STAGING[int(re.search(r"KTileILi(\d+)", name).group(1))]
        start = lines.index("s_nop 4")                    # the prelude's first line
        end = lines.index("s_barrier", start)             # the loop statement's barrier
        prelude_loads = 0
        for ins in lines[start:end]:
            if not ins or ins.startswith((".", "s_")):
                continue
            m = re.match(r"buffer_load_dwordx4 v\[(\d+):\d+\], \S+, \S+, \S+ offen$", ins)
            if m and 80 <= int(m.group(1)) <= last:
                prelude_loads += 1
                continue
            touched = [r for r in _registers(ins) if r[1] >= 80 and r[0] <= last]
            assert not touched, (name, ins)
        assert prelude_loads * 4 == last - 80 + 1, name  # every staging register loaded once
