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

from dense_fp32_matrix_row_amd import build as lib_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "dense_fp32_matrix_row_amd", "csrc")
HIPCC = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")


@pytest.fixture(scope="module")
def assembly(tmp_path_factory):
    if not os.path.exists(HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("isa") / "l10_kloop.s"
    cmd = [HIPCC if os.path.exists(HIPCC) else "hipcc", *lib_build.HIPCC_FLAGS, "--cuda-device-only",
           "-S", lib_build.KLOOP_SOURCE, "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True, timeout=600)
    return out.read_text()


def test_staging_registers_untouched_between_prelude_and_loop(assembly):
    """The check the build runs before linking passes on the sources."""
    assert lib_build.check_kloop_staging(assembly) == []


def test_check_rejects_a_staging_copy(assembly):
    """A copy of a staging register placed between the two statements, or a
    missing prelude load, is reported (planted in the assembly text)."""
    name, lines = next(lib_build.kloop_kernels(assembly))
    start = assembly.index("s_nop 4", assembly.index(name + ":"))
    planted = assembly[:start] + "s_nop 4\n\tv_mov_b32 v3, v81\n" + assembly[start + len("s_nop 4"):]
    bad = lib_build.check_kloop_staging(planted)
    assert bad and "staging register" in bad[0][1]
    load = re.search(r"buffer_load_dwordx4 v\[8[0-9]:\d+\][^\n]*offen\n", assembly[start:])
    dropped = assembly[:start + load.start()] + assembly[start + load.end():]
    assert any("prelude loads" in why for _, why in lib_build.check_kloop_staging(dropped))
