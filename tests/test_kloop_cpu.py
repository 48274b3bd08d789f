"""Host-side checks of the assembly K loop of l10_kloop.hip (no GPU).

The loop text is emitted by gen_kloop.py; the committed l10_kloop.inc must
be exactly that output.  Its LDS traffic is then replayed on the CPU from
the emitted instructions themselves (their immediate offsets) and the
kernel's per-thread base addresses, restated here from l10_kloop.hip:
every access must stay inside the block's LDS allocation and inside its
operand's region, and the word each MFMA operand read finds must be the one
the stage stores put there for that (row, k) or (k, column) -- the loop's
layout is consistent with the operand map the epilogue assumes.
"""

from __future__ import annotations

import importlib.util
import os
import re

import pytest

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                    "dense_fp32_matrix_row_amd", "csrc")


def _gen():
    spec = importlib.util.spec_from_file_location("gen_kloop", os.path.join(CSRC, "gen_kloop.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


G = _gen()
LDS = 2 * G.A_STAGE + 2 * G.B_STAGE
A_END = 2 * G.A_STAGE


def test_committed_loop_matches_generator():
    with open(os.path.join(CSRC, "l10_kloop.inc")) as f:
        assert f.read() == G.render()


# Base addresses (bytes) of l10_kloop.hip, per thread tid = 64 wave + lane.
def w_a(tid):
    return ((tid % 4) * G.A_GROUP + tid // 4) * 4


def w_b(tid):
    return A_END + tid * 16


def r_a(tid):
    wave, lane = divmod(tid, 64)
    return ((lane // 16) * G.BM + (wave // 2) * 64 + 4 * (lane % 16)) * 4


def r_b(tid):
    wave, lane = divmod(tid, 64)
    return A_END + ((lane // 16) * G.BN + (wave % 2) * 64 + 4 * (lane % 16)) * 4


def _stage_stores(buf):
    """{byte address: ('A', row, k) or ('B', k, col)} written by one stage's
    stores into buffer buf, replayed from the emitted instructions."""
    written = {}
    lines = G.stage_stores(buf)
    a_lines = [l for l in lines if l.startswith("ds_write2st64_b32")]
    b_lines = [l for l in lines if l.startswith("ds_write_b128")]
    assert len(a_lines) == 4 and len(b_lines) == 1
    for tid in range(512):
        # the two A float4s: v[80:83] row tid/4, v[84:87] row tid/4 + 128,
        # component c is k = 4 (tid % 4) + c
        regs = {}
        for h in range(2):
            for c in range(4):
                regs[80 + 4 * h + c] = ("A", tid // 4 + 128 * h, 4 * (tid % 4) + c)
        for line in a_lines:
            m = re.match(r"ds_write2st64_b32 %\[wA\], v(\d+), v(\d+) offset0:(\d+) offset1:(\d+)", line)
            r0, r1, o0, o1 = (int(x) for x in m.groups())
            for reg, off in ((r0, o0), (r1, o1)):
                addr = w_a(tid) + 256 * off
                assert 0 <= addr and addr + 4 <= A_END, (tid, line)
                assert addr not in written, ("store overlap", tid, line)
                written[addr] = regs[reg]
        m = re.match(r"ds_write_b128 %\[wB\], v\[88:91\] offset:(\d+)", b_lines[0])
        base = w_b(tid) + int(m.group(1))
        for c in range(4):
            addr = base + 4 * c
            assert A_END <= addr and addr + 4 <= LDS, tid
            assert addr not in written
            written[addr] = ("B", tid // 32, 4 * (tid % 32) + c)
    return written


def test_first_stage_map_matches_the_loop():
    """Stage 0 is stored by the kernel's C++ part (A word (tid % 4) * A_GROUP
    + tid / 4 + 128 h + 256 c, B float4 at word 4 tid of the B region, both
    as in l10_kloop.hip) into buffer 0: it must put every element where the
    loop's own stores into buffer 0 put it."""
    written = _stage_stores(0)
    for tid in range(512):
        for h in range(2):
            for c in range(4):
                word = (tid % 4) * G.A_GROUP + tid // 4 + 128 * h + G.BM * c
                assert written[4 * word] == ("A", tid // 4 + 128 * h, 4 * (tid % 4) + c)
        for c in range(4):
            assert written[A_END + 16 * tid + 4 * c] == ("B", tid // 32, 4 * (tid % 32) + c)


@pytest.mark.parametrize("buf", [0, 1])
def test_fragment_reads_find_their_operands(buf):
    written = _stage_stores(buf)
    # a whole stage lands: 256 x 16 A words and 16 x 128 B words
    assert len(written) == 256 * 16 + 16 * 128
    for s in range(4):
        lines = G.frag_reads(64, s, buf)
        offs = [int(re.search(r"offset:(\d+)", l).group(1)) for l in lines]
        for tid in range(512):
            wave, lane = divmod(tid, 64)
            wm, wn, lrow, kg = wave // 2, wave % 2, lane % 16, lane // 16
            k = 4 * s + kg
            for e in range(4):
                a_addr = r_a(tid) + offs[0] + 4 * e
                b_addr = r_b(tid) + offs[1] + 4 * e
                assert 0 <= a_addr and a_addr + 4 <= A_END
                assert A_END <= b_addr and b_addr + 4 <= LDS
                # block e of the lane: A row 4 lrow + e, B column 4 lrow + e
                assert written[a_addr] == ("A", wm * 64 + 4 * lrow + e, k), (s, tid, e)
                assert written[b_addr] == ("B", k, wn * 64 + 4 * lrow + e), (s, tid, e)


def test_loop_structure():
    prog = G.program()
    mfmas = [l for l in prog if l.startswith("v_mfma")]
    # the prologue issues no MFMA; a pair of K steps and the odd step: 3 x 64
    assert len(mfmas) == 3 * 64
    # every accumulator block gets exactly four MFMAs per K step, one per step s
    for b in range(16):
        assert sum(1 for l in mfmas if l.startswith(f"v_mfma_f32_16x16x4_f32 v[{4*b}:")) == 12
    # each stage: one barrier per K step, plus the prologue's
    assert sum(1 for l in prog if l == "s_barrier") == 4
    # no instruction of the loop writes memory other than LDS
    assert all(not l.startswith(("buffer_store", "global_store", "flat_store")) for l in prog)
