"""Host-side replay of every global-memory load of the assembly K loops of
l10_kloop.hip (no GPU), for each tile and operand orientation gen_kloop.py
builds a loop for.

The loops read A and B with raw buffer loads: a 128-bit resource (base
address, record count in bytes) in SGPRs, a per-thread byte offset in a
VGPR, and a scalar offset.  A load whose offset reaches the record count
returns zeros without touching memory; for a 128-bit load each dword is
checked on its own.  Whether the scalar offset takes part in that check is
not relied on: the replay checks every load under both readings (scalar
offset inside the check, and outside it), and requires each dword a load
could fetch to lie inside its operand's extent (first element to last
element as stored, row padding included), so that a caller whose matrix
ends at the end of a mapped page can never see a fault.

The replay executes the emitted prelude and loop text itself (loads, the
scalar arithmetic that advances the resources, the loop counter and its
branches), with the per-thread offsets and the initial scalar state
restated from l10_kloop.hip, over whole, ragged-K, tiny-K, edge, padded
and split-K problems.  It also checks that every stage the MFMAs consume
holds the elements the k-major layout expects: loaded from their own
addresses for rows and columns inside the tile, and that the loop issues
exactly the stages it needs plus its prefetch.  The 256 x 128 tile's fringe
variant also loads, per stage, one element of the row below the tile and
one of the column right of it (record counts one row / column longer where
the block has that fringe): those loads are replayed the same way, over
grids with and without the extra row and column.
"""

from __future__ import annotations

import importlib.util
import os
import re

import numpy as np
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
MASK32 = 0xFFFFFFFF

# Operand start addresses for the replay: low words at several distances
# below a 2^32 wrap, so that an advance that forgets the carry into the high
# word shows whatever the stage's stride.
ADDRS = [(0x7F12_FFFF_FF00, 0x7E34_FFFF_FE00), (0x7F12_FFFF_FFE0, 0x7E34_FFFF_FFC0),
         (0x7F12_FFFF_0000, 0x7E34_FFFF_8000)]


def slot(tid, per, transposing):
    """(major, four-wide group) of thread tid's first float4: a half-
    wavefront of a transposing 64-deep stage (per 16) takes 4 majors x 8
    groups, every other stage consecutive groups of one major."""
    if transposing and per == 16:
        return 4 * (tid // 64) + (tid // 8) % 4, tid % 8 + 8 * ((tid // 32) % 2)
    return tid // per, tid % per


def a_map(t, tid, h):
    """(row, k) of the first element of float4 h of thread tid (A as
    stored: row-major, four k per float4; transposed, four rows)."""
    per = t.BM // 4 if t.TA else t.BK // 4
    j, q = slot(tid, per, not t.TA)
    major, minor = j + h * (t.THREADS // per), 4 * q
    return (minor, major) if t.TA else (major, minor)


def b_map(t, tid, h):
    """(k, column) of the first element of float4 h of thread tid."""
    per = t.BK // 4 if t.TB else t.BN // 4
    j, q = slot(tid, per, t.TB)
    major, minor = j + h * (t.THREADS // per), 4 * q
    return (minor, major) if t.TB else (major, minor)


class Problem:
    """One work item's view of a problem, restated from k_kloop: the tile
    at (row0, col0), K part [k_lo, k_lo + kp)."""

    def __init__(self, t, M, N, K, lda, ldb, row0, col0, k_lo=0, kp=None, addrs=ADDRS[0], grid=None):
        self.t, self.M, self.N, self.K, self.lda, self.ldb = t, M, N, K, lda, ldb
        self.addr_a, self.addr_b = addrs
        self.row0, self.col0, self.k_lo = row0, col0, k_lo
        self.kp = K - k_lo if kp is None else kp
        self.rows = min(M - row0, t.BM)
        self.cols = min(N - col0, t.BN)
        # fringe variant over a grid of Mm x Nm whole tiles: row M - 1 /
        # column N - 1 beside it, which every block reads
        Mm, Nm = grid if grid else (M, N)
        self.f_row = t.FRINGE and M == Mm + 1
        self.f_col = t.FRINGE and N == Nm + 1
        self.a_last = M - 1 - row0 if self.f_row else self.rows - 1
        self.b_last = N - 1 - col0 if self.f_col else self.cols - 1
        # strides of A (m, k) and B (k, n) as stored, in elements
        self.a_rs, self.a_ks = (1, lda) if t.TA else (lda, 1)
        self.b_ks, self.b_cs = (1, ldb) if t.TB else (ldb, 1)
        # operand extents: first to last element as stored
        self.a_end = self.addr_a + 4 * (((K - 1) * lda + M) if t.TA else ((M - 1) * lda + K))
        self.b_end = self.addr_b + 4 * (((N - 1) * ldb + K) if t.TB else ((K - 1) * ldb + N))
        self.k0 = self.kp % t.BK or t.BK
        self.stages = -(-self.kp // t.BK)

    def initial_state(self):
        """SGPRs and named asm operands at the prelude, as the kernel sets
        them: resources based at the tile's first element of stage 1, with
        record counts that end at the tile's last element (never negative)."""
        t = self.t
        a_base = self.addr_a + 4 * (self.row0 * self.a_rs + self.k_lo * self.a_ks)
        b_base = self.addr_b + 4 * (self.col0 * self.b_cs + self.k_lo * self.b_ks)
        a_bytes = 4 * (self.a_last * self.a_rs + (self.kp - 1) * self.a_ks + 1)
        b_bytes = 4 * ((self.kp - 1) * self.b_ks + self.b_last * self.b_cs + 1)
        a_skip, b_skip = 4 * self.k0 * self.a_ks, 4 * self.k0 * self.b_ks
        sg = {}
        for reg, base, nrec in ((G.RES_A, a_base + a_skip, max(a_bytes - a_skip, 0)),
                                (G.RES_B, b_base + b_skip, max(b_bytes - b_skip, 0))):
            sg[reg] = base & MASK32
            sg[reg + 1] = (base >> 32) & 0xFFFF
            sg[reg + 2] = nrec
            sg[reg + 3] = 0x00020000
        ops = {"stepA": 4 * t.BK * self.a_ks, "stepB": 4 * t.BK * self.b_ks,
               "pairs": self.stages // 2, "odd": self.stages % 2}
        return sg, ops

    def offsets(self):
        """Per-thread byte offsets {('A', h): array over tid} (VGPR inputs)."""
        t, tid = self.t, np.arange(self.t.THREADS)
        out = {}
        for h in range(t.A_LOADS):
            r, k = a_map(t, tid, h)
            out[("A", h)] = 4 * (r * self.a_rs + k * self.a_ks)
        for h in range(t.B_LOADS):
            k, c = b_map(t, tid, h)
            out[("B", h)] = 4 * (k * self.b_ks + c * self.b_cs)
        if t.FRINGE:
            # element (a_last, k) of the tile's A and (k, b_last) of its B,
            # k = tid % BK: row M - 1 / column N - 1 where they exist
            out[("FA", 0)] = 4 * (self.a_last * self.a_rs + (tid % t.BK) * self.a_ks)
            out[("FB", 0)] = 4 * ((tid % t.BK) * self.b_ks + self.b_last * self.b_cs)
        return out


LOAD = re.compile(r"buffer_load_dwordx4 v\[(\d+):(\d+)\], %\[o([AB])(\d)\], s\[(\d+):(\d+)\], (\S+) offen$")
LOAD_F = re.compile(r"buffer_load_dword v(\d+), %\[fo([ab])\], s\[(\d+):(\d+)\], (\S+) offen$")
SALU3 = re.compile(r"(s_add_u32|s_addc_u32|s_sub_u32|s_cselect_b32|s_min_u32) (\S+), (\S+), (\S+)$")
SCMP = re.compile(r"(s_cmp_eq_u32|s_cmp_lg_u32) (\S+), (\S+)$")


def execute(t, sg, ops):
    """Run the prelude, then the loop, on the scalar state; return the load
    events in issue order: (operand, h, base, record count, scalar offset)."""
    state = {"scc": 0}

    def val(tok):
        if tok.startswith("%["):
            return ops[tok[2:-1]]
        if re.fullmatch(r"s\d+", tok):
            return sg[int(tok[1:])]
        return int(tok, 0)

    def put(tok, v):
        if tok.startswith("%["):
            ops[tok[2:-1]] = v & MASK32
        else:
            sg[int(tok[1:])] = v & MASK32

    events = []
    for prog in (t.prelude(), t.program()):
        labels = {l[:-1]: i for i, l in enumerate(prog) if l.endswith(":")}
        pc, executed = 0, 0
        while pc < len(prog):
            ins = prog[pc]
            pc += 1
            executed += 1
            assert executed < 10_000_000
            m = LOAD.match(ins)
            if m:
                lo, hi = int(m.group(5)), int(m.group(6))
                assert hi == lo + 3 and lo % 4 == 0, ins
                base = sg[lo] | ((sg[lo + 1] & 0xFFFF) << 32)
                events.append((m.group(3), int(m.group(4)), base, sg[lo + 2], val(m.group(7))))
                continue
            m = LOAD_F.match(ins)
            if m:
                lo, hi = int(m.group(3)), int(m.group(4))
                assert hi == lo + 3 and lo % 4 == 0, ins
                base = sg[lo] | ((sg[lo + 1] & 0xFFFF) << 32)
                events.append(("F" + m.group(2).upper(), 0, base, sg[lo + 2], val(m.group(5))))
                continue
            m = SALU3.match(ins)
            if m:
                op, d, a, b = m.groups()
                x, y = val(a), val(b)
                if op == "s_add_u32":
                    r = x + y
                    state["scc"] = int(r > MASK32)
                elif op == "s_addc_u32":
                    r = x + y + state["scc"]
                    state["scc"] = int(r > MASK32)
                elif op == "s_sub_u32":
                    r = x - y
                    state["scc"] = int(y > x)
                elif op == "s_cselect_b32":
                    r = x if state["scc"] else y
                else:
                    r = min(x, y)
                    state["scc"] = int(x < y)
                put(d, r)
                continue
            m = SCMP.match(ins)
            if m:
                op, a, b = m.groups()
                state["scc"] = int((val(a) == val(b)) == (op == "s_cmp_eq_u32"))
                continue
            if ins.startswith("s_cbranch_scc1 "):
                if state["scc"]:
                    pc = labels[ins.split()[1]]
                continue
            assert not ins.startswith(("buffer_", "global_", "flat_", "s_load", "s_buffer")), ins
            assert not re.match(r"s_\w+ s\d+", ins) or ins.startswith(("s_waitcnt", "s_nop")), \
                f"scalar instruction the replay does not model: {ins}"
    return events


def replay(p: Problem):
    t = p.t
    sg, ops = p.initial_state()
    offs = p.offsets()
    events = execute(t, sg, ops)
    per_stage = t.A_LOADS + t.B_LOADS + (2 if t.FRINGE else 0)
    # stages 1 .. stages - 1 are requested once each, and DEPTH + 1 past the
    # last (every step requests the stage DEPTH + 1 ahead of it)
    assert len(events) == per_stage * (p.stages + t.DEPTH), (len(events), p.stages)
    for i, (op, h, base, nrec, soff) in enumerate(events):
        stage = 1 + i // per_stage
        comp = 4 * np.arange(1 if op in ("FA", "FB") else 4)
        off = offs[(op, h)][:, None] + comp[None, :]          # (threads, 4) bytes
        addr = base + soff + off
        lo, hi = (p.addr_a, p.a_end) if op in ("A", "FA") else (p.addr_b, p.b_end)
        inside = (addr >= lo) & (addr + 4 <= hi)
        for performed in (off + 4 <= nrec, soff + off + 4 <= nrec):
            bad = performed & ~inside
            assert not bad.any(), (t.name, op, h, stage, hex(int(addr[bad][0])), hex(lo), hex(hi))
        if stage >= p.stages:
            continue  # prefetch past the last stage: lands in LDS unused
        # consumed stage: in-tile elements must come from their own address
        tid = np.arange(t.THREADS)
        kbase = p.k_lo + p.k0 + (stage - 1) * t.BK
        if op in ("FA", "FB"):
            # where the grid has the fringe, the element of k = tid % BK of
            # row M - 1 / column N - 1, for every k of the stage below K
            kk = (tid % t.BK)[:, None]
            if op == "FA":
                want = p.addr_a + 4 * ((p.M - 1) * p.a_rs + (kbase + kk) * p.a_ks)
                has = p.f_row
            else:
                want = p.addr_b + 4 * ((kbase + kk) * p.b_ks + (p.N - 1) * p.b_cs)
                has = p.f_col
            if has:
                assert (kbase + kk < p.k_lo + p.kp).all()
                for performed in (off + 4 <= nrec, soff + off + 4 <= nrec):
                    assert performed.all(), (t.name, op, stage, "fringe element not loaded")
                assert (addr == want).all(), (t.name, op, stage, "wrong fringe element")
            continue
        if op == "A":
            r, k = a_map(t, tid, h)
            rr = r[:, None] + (comp[None, :] // 4 if t.TA else 0)
            kk = k[:, None] + (0 if t.TA else comp[None, :] // 4)
            want = p.addr_a + 4 * ((p.row0 + rr) * p.a_rs + (kbase + kk) * p.a_ks)
            need = rr < p.rows
        else:
            k, c = b_map(t, tid, h)
            kk = k[:, None] + (comp[None, :] // 4 if t.TB else 0)
            cc = c[:, None] + (0 if t.TB else comp[None, :] // 4)
            want = p.addr_b + 4 * ((kbase + kk) * p.b_ks + (p.col0 + cc) * p.b_cs)
            need = cc < p.cols
        need = np.broadcast_to(need, addr.shape)
        assert (kbase + kk < p.k_lo + p.kp).all()
        for performed in (off + 4 <= nrec, soff + off + 4 <= nrec):
            assert (performed | ~need).all(), (t.name, op, h, stage, "in-tile element not loaded")
        assert (addr == want)[need].all(), (t.name, op, h, stage, "wrong element")


def _problems(t):
    """(M, N, K, lda, ldb, k_split) cases for tile t; op(A) is M x K, op(B)
    K x N, stored transposed where the tile says so."""
    BM, BN, BK = t.BM, t.BN, t.BK
    cases = [
        (2 * BM, 2 * BN, 4 * BK, None),      # whole tiles, K a multiple of the stage
        (2 * BM, BN, 3 * BK + 5, None),      # ragged K
        (BM, BN, 1, None),                   # K of one element
        (BM, BN, BK, None),                  # one whole stage: the prelude loads past K
        (BM, BN, BK + 1, None),
        (BM + 17, BN + 3, 2 * BK + 3, None),  # bottom / right edge tiles
        (BM - 5, BN - 9, 5 * BK, None),       # a single partial tile
        (2 * BM, 2 * BN, 7 * BK + 2, 2 * BK),  # split K, last part short
        (BM + 1, BN + 1, 6 * BK, 3 * BK),      # split K over edge tiles
    ]
    out = []
    for M, N, K, ks in cases:
        ld_a = M if t.TA else K
        ld_b = K if t.TB else N
        out.append((M, N, K, ld_a, ld_b, ks))          # packed
        out.append((M, N, K, ld_a + 7, ld_b + 5, ks))  # padded rows
    return out


def _fringe_problems(t):
    """(Mm, Nm, M, N, K, lda, ldb) cases for the fringe variant: whole tiles
    over the first Mm x Nm of C (at least as many as the variant takes:
    shares of at most THREADS / BK), and one more row and / or column."""
    BM, BN, BK = t.BM, t.BN, t.BK
    fp = t.THREADS // BK
    mt, nt = -(-BN // fp), -(-BM // fp)
    out = []
    for Mm, Nm, K in [(mt * BM, nt * BN, 4 * BK), ((mt + 1) * BM, nt * BN, 3 * BK + 5), (mt * BM, (nt + 1) * BN, 1),
                      (mt * BM, nt * BN, BK), (mt * BM, nt * BN, BK + 1), (mt * BM, nt * BN, 5 * BK + 15)]:
        for dm, dn in ((1, 1), (1, 0), (0, 1)):
            M, N = Mm + dm, Nm + dn
            ld_a = M if t.TA else K
            ld_b = K if t.TB else N
            out.append((Mm, Nm, M, N, K, ld_a, ld_b))
            out.append((Mm, Nm, M, N, K, ld_a + 7, ld_b + 5))
    return out


@pytest.mark.parametrize("name", sorted(TILES))
def test_global_loads_stay_inside_their_operands(name):
    t = TILES[name]
    if t.FRINGE:
        # the grid's tiles only (the kernel's grid): its corners and an
        # inner one, every block reading row M - 1 / column N - 1
        for Mm, Nm, M, N, K, lda, ldb in _fringe_problems(t):
            lm, ln = Mm - t.BM, Nm - t.BN
            for row0, col0 in [(0, 0), (0, ln), (lm, 0), (lm, ln), (t.BM, 2 * t.BN)]:
                for addrs in ADDRS:
                    replay(Problem(t, M, N, K, lda, ldb, row0, col0, 0, K, addrs, grid=(Mm, Nm)))
        return
    for M, N, K, lda, ldb, ks in _problems(t):
        parts = [(0, K)] if ks is None else [(lo, min(ks, K - lo)) for lo in range(0, K, ks)]
        for row0 in range(0, M, t.BM):
            for col0 in range(0, N, t.BN):
                for k_lo, kp in parts:
                    for addrs in ADDRS:
                        replay(Problem(t, M, N, K, lda, ldb, row0, col0, k_lo, kp, addrs))


def test_resource_registers_are_the_pinned_ones():
    """The loop text names the resource quads the kernel pins (l10_kloop.hip
    binds them with the same register constraints)."""
    src = open(os.path.join(CSRC, "l10_kloop.hip")).read()
    for reg in (G.RES_A, G.RES_B):
        assert f"{{s[{reg}:{reg + 3}]}}" in src
    for t in G.TILES:
        for ins in t.prelude() + t.program():
            if ins.startswith("buffer_load"):
                assert f"s[{G.RES_A}:{G.RES_A + 3}], 0 offen" in ins or \
                       f"s[{G.RES_B}:{G.RES_B + 3}], 0 offen" in ins, ins
