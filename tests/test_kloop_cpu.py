"""Host-side checks of the assembly K loops of l10_kloop.hip (no GPU), for
each tile gen_kloop.py builds a loop for.

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
TILES = {t.name: t for t in G.TILES}


def test_committed_loop_matches_generator():
    with open(os.path.join(CSRC, "l10_kloop.inc")) as f:
        assert f.read() == G.render()


# Base addresses (bytes) of l10_kloop.hip, per thread tid = 64 wave + lane.
def w_a(t, tid):
    return ((tid % 4) * t.A_GROUP + tid // 4) * 4


def w_b(t, tid):
    return 2 * t.A_STAGE + tid * 16


def _wave(t, tid):
    """(wm, wn, lrow, kg) of a thread."""
    wave, lane = divmod(tid, 64)
    return wave // 2, wave % 2, lane % 16, lane // 16


def r_a(t, tid):
    wm, _, lrow, kg = _wave(t, tid)
    return (kg * t.BM + wm * 64 + 4 * lrow) * 4


def r_b(t, tid):
    _, wn, lrow, kg = _wave(t, tid)
    return 2 * t.A_STAGE + (kg * G.BN + wn * 64 + 4 * lrow) * 4


def _stage_stores(t, st, buf):
    """{byte address: ('A', row, k) or ('B', k, col)} written by one stage's
    stores from staging set st into buffer buf, replayed from the emitted
    instructions."""
    written = {}
    a_end = 2 * t.A_STAGE
    base = t.set_base(st)
    lines = t.stage_stores(st, buf)
    a_lines = [l for l in lines if l.startswith("ds_write2st64_b32")]
    b_lines = [l for l in lines if l.startswith("ds_write_b128")]
    assert len(a_lines) == 2 * t.A_LOADS and len(b_lines) == t.B_LOADS
    for tid in range(t.THREADS):
        # staging words: A float4 h (row tid/4 + h THREADS/4, k = 4 (tid%4) + c),
        # then B float4 h (k-row tid/32 + h THREADS/32, columns 4 (tid%32) + c)
        regs = {}
        for h in range(t.A_LOADS):
            for c in range(4):
                regs[base + 4 * h + c] = ("A", tid // 4 + h * t.THREADS // 4, 4 * (tid % 4) + c)
        for h in range(t.B_LOADS):
            for c in range(4):
                regs[base + 4 * t.A_LOADS + 4 * h + c] = ("B", tid // 32 + h * t.THREADS // 32,
                                                          4 * (tid % 32) + c)
        for line in a_lines:
            m = re.match(r"ds_write2st64_b32 %\[wA\], v(\d+), v(\d+) offset0:(\d+) offset1:(\d+)", line)
            r0, r1, o0, o1 = (int(x) for x in m.groups())
            for reg, off in ((r0, o0), (r1, o1)):
                addr = w_a(t, tid) + 256 * off
                assert 0 <= addr and addr + 4 <= a_end, (tid, line)
                assert addr not in written, ("store overlap", tid, line)
                written[addr] = regs[reg]
        for line in b_lines:
            m = re.match(r"ds_write_b128 %\[wB\], v\[(\d+):(\d+)\] offset:(\d+)", line)
            r0, r3, off = (int(x) for x in m.groups())
            assert r3 == r0 + 3
            for c in range(4):
                addr = w_b(t, tid) + off + 4 * c
                assert a_end <= addr and addr + 4 <= t.LDS, tid
                assert addr not in written
                written[addr] = regs[r0 + c]
    return written


@pytest.mark.parametrize("bm", sorted(TILES))
def test_first_stage_map_matches_the_loop(bm):
    """Stage 0 is stored by the kernel's C++ part (A word (tid % 4) A_GROUP +
    tid / 4 + h THREADS/4 + BM c, B float4 h at word 4 (tid + h THREADS) of
    the B region, both as in l10_kloop.hip) into buffer 0: it must put every
    element where the loop's own stores into buffer 0 put it."""
    t = TILES[bm]
    written = _stage_stores(t, 0, 0)
    a_end = 2 * t.A_STAGE
    for tid in range(t.THREADS):
        for h in range(t.A_LOADS):
            for c in range(4):
                word = (tid % 4) * t.A_GROUP + tid // 4 + h * t.THREADS // 4 + t.BM * c
                assert written[4 * word] == ("A", tid // 4 + h * t.THREADS // 4, 4 * (tid % 4) + c)
        for h in range(t.B_LOADS):
            for c in range(4):
                assert written[a_end + 16 * (tid + h * t.THREADS) + 4 * c] == (
                    "B", tid // 32 + h * t.THREADS // 32, 4 * (tid % 32) + c)


@pytest.mark.parametrize("bm", sorted(TILES))
@pytest.mark.parametrize("buf", [0, 1])
def test_fragment_reads_find_their_operands(bm, buf):
    t = TILES[bm]
    a_end = 2 * t.A_STAGE
    for st in range(t.DEPTH):
        written = _stage_stores(t, st, buf)
        # a whole stage lands: BM x 16 A words and 16 x 128 B words
        assert len(written) == t.BM * 16 + 16 * G.BN
        for s in range(t.STEPS):
            lines = t.frag_reads(64, s, buf)
            offs = [int(re.search(r"offset:(\d+)", l).group(1)) for l in lines]
            for tid in range(t.THREADS):
                wm, wn, lrow, kg = _wave(t, tid)
                k = 4 * s + kg
                for e in range(4):
                    a_addr = r_a(t, tid) + offs[0] + 4 * e
                    b_addr = r_b(t, tid) + offs[1] + 4 * e
                    assert 0 <= a_addr and a_addr + 4 <= a_end
                    assert a_end <= b_addr and b_addr + 4 <= t.LDS
                    # block e of the lane: A row 4 lrow + e, B column 4 lrow + e
                    assert written[a_addr] == ("A", wm * 64 + 4 * lrow + e, k), (s, tid, e)
                    assert written[b_addr] == ("B", k, wn * 64 + 4 * lrow + e), (s, tid, e)


@pytest.mark.parametrize("bm", sorted(TILES))
def test_loop_structure(bm):
    t = TILES[bm]
    prog = t.program()
    mfmas = [l for l in prog if l.startswith("v_mfma")]
    # the prologue issues no MFMA; a pair of K steps and the odd step: 3 x 64
    assert len(mfmas) == 3 * 64
    # every accumulator block gets exactly four MFMAs per K step, one per step s
    for b in range(16):
        assert sum(1 for l in mfmas if l.startswith(f"v_mfma_f32_16x16x4_f32 v[{4*b}:")) == 12
    # one barrier per K step, plus the prologue's
    assert sum(1 for l in prog if l == "s_barrier") == 4
    # no instruction of the loop writes memory other than LDS
    assert all(not l.startswith(("buffer_store", "global_store", "flat_store")) for l in prog)
    # every register the loop names lies in the pinned range v0 .. last_vgpr
    for l in prog:
        for lo, hi in re.findall(r"v\[(\d+):(\d+)\]", l):
            assert int(hi) <= t.last_vgpr()
        for r in re.findall(r"\bv(\d+)\b", l):
            assert int(r) <= t.last_vgpr()


@pytest.mark.parametrize("bm", sorted(TILES))
def test_staging_sets_are_waited_for_before_their_stores(bm):
    """With DEPTH staging sets, the loop's stores of stage n + 1 follow a
    vmcnt wait that leaves at most the younger DEPTH - 1 stages' loads in
    flight, and each set is reloaded only after an lgkmcnt(0) that follows
    its stores (the stores have read the registers)."""
    t = TILES[bm]
    per_stage = t.A_LOADS + t.B_LOADS
    for cur in (0, 1):
        step = t.k_step(cur)
        first_store = next(i for i, l in enumerate(step) if l.startswith("ds_write"))
        waits = [l for l in step[:first_store] if l.startswith("s_waitcnt vmcnt")]
        assert waits == [f"s_waitcnt vmcnt({per_stage * (t.DEPTH - 1)})"]
        last_store = max(i for i, l in enumerate(step) if l.startswith("ds_write"))
        first_load = next(i for i, l in enumerate(step) if l.startswith("buffer_load"))
        assert "s_waitcnt lgkmcnt(0)" in step[last_store:first_load]
