"""Host-side checks of the assembly K loops of l10_kloop.hip (no GPU), for
each tile and operand orientation gen_kloop.py builds a loop for.

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


# Per-thread element maps and base addresses of l10_kloop.hip (restated from
# the kernel): element h of thread tid is
#   A row-major:  row tid/4 + h THREADS/4, k 4 (tid%4) + c
#   A transposed: k-row tid/(BM/4) + 8 h, row 4 (tid%(BM/4)) + c
#   B row-major:  k-row tid/32 + h THREADS/32, column 4 (tid%32) + c
#   B transposed: column tid/4 + h THREADS/4, k 4 (tid%4) + c
def a_elem(t, tid, h, c):
    if t.TA:
        return ("A", 4 * (tid % (t.BM // 4)) + c, tid // (t.BM // 4) + 8 * h)
    return ("A", tid // 4 + h * t.THREADS // 4, 4 * (tid % 4) + c)


def b_elem(t, tid, h, c):
    if t.TB:
        return ("B", 4 * (tid % 4) + c, tid // 4 + h * t.THREADS // 4)
    return ("B", tid // 32 + h * t.THREADS // 32, 4 * (tid % 32) + c)


def a_word(t, m, k):
    """LDS word of A element (m, k): k-row k at group k/4, word (k%4) BM + m."""
    return (k // 4) * t.A_GROUP + (k % 4) * t.BM + m


def b_word(t, k, n):
    return 2 * t.A_STAGE // 4 + (k // 4) * t.B_GROUP + (k % 4) * G.BN + n


def w_a(t, tid):
    _, m, k = a_elem(t, tid, 0, 0)
    return 4 * a_word(t, m, k)


def w_b(t, tid):
    _, k, n = b_elem(t, tid, 0, 0)
    return 4 * b_word(t, k, n)


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
    instructions (their registers and immediate offsets)."""
    written = {}
    a_end = 2 * t.A_STAGE
    base = t.set_base(st)
    lines = t.stage_stores(st, buf)
    for tid in range(t.THREADS):
        regs = {}
        for h in range(t.A_LOADS):
            for c in range(4):
                regs[base + 4 * h + c] = a_elem(t, tid, h, c)
        for h in range(t.B_LOADS):
            for c in range(4):
                regs[base + 4 * t.A_LOADS + 4 * h + c] = b_elem(t, tid, h, c)
        for line in lines:
            m2 = re.match(r"ds_write2st64_b32 %\[w([AB])\], v(\d+), v(\d+) offset0:(\d+) offset1:(\d+)$", line)
            m4 = re.match(r"ds_write_b128 %\[w([AB])\], v\[(\d+):(\d+)\] offset:(\d+)$", line)
            assert m2 or m4, line
            if m2:
                op, r0, r1, o0, o1 = m2.group(1), *(int(x) for x in m2.groups()[1:])
                pieces = [(r0, 256 * o0), (r1, 256 * o1)]
            else:
                op, r0, r3, off = m4.group(1), *(int(x) for x in m4.groups()[1:])
                assert r3 == r0 + 3
                pieces = [(r0 + c, off + 4 * c) for c in range(4)]
            start = w_a(t, tid) if op == "A" else w_b(t, tid)
            lo, hi = (0, a_end) if op == "A" else (a_end, t.LDS)
            for reg, off in pieces:
                addr = start + off
                assert lo <= addr and addr + 4 <= hi, (t.name, tid, line)
                assert addr not in written, ("store overlap", t.name, tid, line)
                assert regs[reg][0] == op, (t.name, line)
                written[addr] = regs[reg]
    return written


@pytest.mark.parametrize("name", sorted(TILES))
def test_first_stage_map_matches_the_loop(name):
    """Stage 0 is stored by the kernel's C++ part through the same element
    maps into buffer 0 (A (m, k) at word (k/4) A_GROUP + (k%4) BM + m, B
    (k, n) likewise): it must put every element where the loop's own stores
    into buffer 0 put it."""
    t = TILES[name]
    written = _stage_stores(t, 0, 0)
    for tid in range(t.THREADS):
        for h in range(t.A_LOADS):
            for c in range(4):
                e = a_elem(t, tid, h, c)
                assert written[4 * a_word(t, e[1], e[2])] == e
        for h in range(t.B_LOADS):
            for c in range(4):
                e = b_elem(t, tid, h, c)
                assert written[4 * b_word(t, e[1], e[2])] == e


@pytest.mark.parametrize("name", sorted(TILES))
@pytest.mark.parametrize("buf", [0, 1])
def test_fragment_reads_find_their_operands(name, buf):
    t = TILES[name]
    a_end = 2 * t.A_STAGE
    for st in range(t.DEPTH):
        written = _stage_stores(t, st, buf)
        # a whole stage lands: BM x 16 A words and 16 x 128 B words
        assert len(written) == t.BM * 16 + 16 * G.BN
        for s in range(4):
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


def _bank_conflict_free_32bit(addrs):
    """The 32 words of one half-wavefront's 32-bit write lie in 32 different
    banks (bank = word mod 64)."""
    return len({(a // 4) % 64 for a in addrs}) == len(addrs)


@pytest.mark.parametrize("name", sorted(TILES))
def test_transposing_stores_hit_distinct_banks(name):
    """Each half-wavefront of a 32-bit transposing store writes 32 different
    banks (the padded groups' purpose)."""
    t = TILES[name]
    for line in t.stage_stores(0, 0):
        m2 = re.match(r"ds_write2st64_b32 %\[w([AB])\], v\d+, v\d+ offset0:(\d+) offset1:\d+$", line)
        if not m2:
            continue
        op, o0 = m2.group(1), int(m2.group(2))
        for first in range(0, t.THREADS, 32):
            addrs = [(w_a(t, tid) if op == "A" else w_b(t, tid)) + 256 * o0 for tid in range(first, first + 32)]
            assert _bank_conflict_free_32bit(addrs), (name, line, first)


@pytest.mark.parametrize("name", sorted(TILES))
def test_loop_structure(name):
    t = TILES[name]
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


@pytest.mark.parametrize("name", sorted(TILES))
def test_staging_sets_are_waited_for_before_their_stores(name):
    """With DEPTH staging sets, the loop's stores of stage n + 1 follow a
    vmcnt wait that leaves at most the younger DEPTH - 1 stages' loads in
    flight, and each set is reloaded only after an lgkmcnt(0) that follows
    its stores (the stores have read the registers)."""
    t = TILES[name]
    per_stage = t.A_LOADS + t.B_LOADS
    for cur in (0, 1):
        step = t.k_step(cur)
        first_store = next(i for i, l in enumerate(step) if l.startswith("ds_write"))
        waits = [l for l in step[:first_store] if l.startswith("s_waitcnt vmcnt")]
        assert waits == [f"s_waitcnt vmcnt({per_stage * (t.DEPTH - 1)})"]
        last_store = max(i for i, l in enumerate(step) if l.startswith("ds_write"))
        first_load = next(i for i, l in enumerate(step) if l.startswith("buffer_load"))
        assert "s_waitcnt lgkmcnt(0)" in step[last_store:first_load]
