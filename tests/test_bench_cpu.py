"""bench.py's host logic without a GPU: the one-GPU guard, the source digest
that decides whether recorded hardware counters still apply, and the
reading of a recorded traffic figure."""

from __future__ import annotations

import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    proc = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                          capture_output=True, text=True, timeout=120)
    assert proc.returncode == 2
    assert "one GPU" in proc.stderr and proc.stdout == ""


def test_code_only_drops_comments_and_keeps_literals():
    text = ('int a = 1;  // a comment\n'
            '/* block\n   comment */ const char* s = "// not a comment /* nor this */";\n'
            '\n'
            "char q = '\"';  /* trailing */\n"
            'asm("s_nop 0\\n" "v_mov_b32 v0, v1\\n");\n')
    assert bench._code_only(text) == ('int a = 1;\n'
                                     ' const char* s = "// not a comment /* nor this */";\n'
                                     "char q = '\"';\n"
                                     'asm("s_nop 0\\n" "v_mov_b32 v0, v1\\n");')
    # a changed comment is the same code; a changed token is not
    assert bench._code_only(text.replace("// a comment", "// another remark")) == bench._code_only(text)
    assert bench._code_only(text.replace("int a = 1", "int a = 2")) != bench._code_only(text)


def test_digest_is_of_the_package_sources():
    d = bench.kernel_source_digest()
    assert len(d) == 16 and int(d, 16) >= 0
    assert d == bench.kernel_source_digest()


def test_recorded_traffic_only_for_the_current_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.recorded_traffic("sgemm_4096", "L10_shape_dispatch") is None  # no file
    path = tmp_path / "pmc_traffic_L10_shape_dispatch_sgemm_4096.txt"
    path.write_text("# kernel = x\nhbm_bytes_per_launch = 672628498\n"
                    f"kernel_source_digest = {bench.kernel_source_digest()}\n")
    assert bench.recorded_traffic("sgemm_4096", "L10_shape_dispatch") == 672628498.0
    path.write_text("hbm_bytes_per_launch = 672628498\nkernel_source_digest = 0000000000000000\n")
    assert bench.recorded_traffic("sgemm_4096", "L10_shape_dispatch") is None
