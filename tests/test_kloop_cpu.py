"""Host-side checks of the assembly K loops of l10_kloop.hip (no GPU), for
each tile and operand orientation gen_kloop.py builds a loop for.

The loop text is emitted by gen_kloop.py; the committed l10_kloop.inc must
be exactly that output.  Its LDS traffic is then replayed on the CPU from
the emitted instructions themselves (their registers and immediate offsets)
and the kernel's per-thread element maps and base addresses, restated here
from l10_kloop.hip: every access must stay inside the block's LDS
allocation and inside its operand's region, every stage store must land
where the k-major layout puts its element, and the word each MFMA operand
read finds must be the one stored there for that (row, k) or (k, column) --
the loop's layout is consistent with the operand map the epilogue assumes.
For the 256 x 128 tile's fringe variant the same replay follows the staged
words of the extra row and column and every FMA of the fringe sums: each
multiplies the extra row's k with B's (k, column), or A's (row, k) with the
extra column's k, for the block's share of columns and rows, and the sums
of a share cover every k of a stage exactly once; the blocks' shares cover
the extra row's and column's outputs exactly once.
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


# Per-thread element maps of l10_kloop.hip (restated from the kernel):
# element h, component c of thread tid, with per = float4s per row (k-row)
# of the operand as stored and (j, q) the thread's slot:
#   A row-major:  row j + h THREADS/per, k 4 q + c
#   A transposed: k-row j + h THREADS/per, row 4 q + c
#   B row-major:  k-row j + h THREADS/per, column 4 q + c
#   B transposed: column j + h THREADS/per, k 4 q + c
# where a transposing store (row-major A, transposed B) with per == 16 puts
# 4 majors x 8 groups in each half-wavefront and every other store
# (j, q) = (tid / per, tid % per).
def slot(tid, per, transposing):
    if transposing and per == 16:
        return 4 * (tid // 64) + (tid // 8) % 4, tid % 8 + 8 * ((tid // 32) % 2)
    return tid // per, tid % per


def a_elem(t, tid, h, c):
    per = t.BM // 4 if t.TA else t.BK // 4
    j, q = slot(tid, per, not t.TA)
    major, minor = j + h * (t.THREADS // per), 4 * q + c
    return ("A", minor, major) if t.TA else ("A", major, minor)


def b_elem(t, tid, h, c):
    per = t.BK // 4 if t.TB else t.BN // 4
    j, q = slot(tid, per, t.TB)
    major, minor = j + h * (t.THREADS // per), 4 * q + c
    return ("B", minor, major) if t.TB else ("B", major, minor)


def a_word(t, m, k):
    """LDS word of A element (m, k): k-row k at group k/4, word (k%4) BM + m."""
    return (k // 4) * t.A_GROUP + (k % 4) * t.BM + m


def b_word(t, k, n):
    return 2 * t.A_STAGE // 4 + (k // 4) * t.B_GROUP + (k % 4) * t.BN + n


def w_a(t, tid):
    _, m, k = a_elem(t, tid, 0, 0)
    return 4 * a_word(t, m, k)


def w_b(t, tid):
    _, k, n = b_elem(t, tid, 0, 0)
    return 4 * b_word(t, k, n)


# The fringe variant's per-block shares and per-thread LDS bases (restated
# from l10_kloop.hip).  Block (i, j) of a tiles_m x tiles_n grid takes
# columns i cpt .. of its tile for the extra row, cpt = ceil(BN / tiles_m),
# and rows j rpt .. for the extra column, rpt = ceil(BM / tiles_n); thread
# tid multiplies k = tid / FP of each stage (FP = THREADS / BK) for share
# position tid % FP (positions beyond the share, or beyond the tile, take
# column / row tid % FP, whose sums are not stored); its staged words are
# those of k = tid / FP (%[fpk]) and, for the corner, of k = tid % BK
# (%[fst]).
def f_share(t, tiles_m, tiles_n, i, j):
    cpt, rpt = -(-t.BN // tiles_m), -(-t.BM // tiles_n)
    return cpt, rpt, i * cpt, j * rpt


def f_cols(t, grid, tid):
    """(column n, row m) of the tile that thread tid's fringe sums take."""
    cpt, rpt, n0, m0 = f_share(t, *grid)
    c = tid % t.FP
    n = n0 + c if c < cpt and n0 + c < t.BN else c
    m = m0 + c if c < rpt and m0 + c < t.BM else c
    return n, m


def f_st(t, grid, tid):
    return 4 * (tid % t.BK)


def f_pk(t, grid, tid):
    return 4 * (tid // t.FP)


def f_rb(t, grid, tid):
    k, (n, _) = tid // t.FP, f_cols(t, grid, tid)
    return 2 * t.A_STAGE + ((k // 4) * t.B_GROUP + (k % 4) * t.BN + n) * 4


def f_ca(t, grid, tid):
    k, (_, m) = tid // t.FP, f_cols(t, grid, tid)
    return ((k // 4) * t.A_GROUP + (k % 4) * t.BM + m) * 4


def f_min_grid(t):
    """Fewest tile rows and columns the variant takes (shares <= FP)."""
    return -(-t.BN // t.FP), -(-t.BM // t.FP)


F_BASES = {"fst": f_st, "frB": f_rb, "fcA": f_ca, "fpk": f_pk}


def _wave(t, tid):
    """(K slice, wm, wn, lrow, kg) of a thread."""
    wave, lane = divmod(tid, 64)
    slice_, wv = divmod(wave, t.WAVES_M * t.WAVES_N)
    return slice_, wv // t.WAVES_N, wv % t.WAVES_N, lane % 16, lane // 16


def r_a(t, tid):
    slice_, wm, _, lrow, kg = _wave(t, tid)
    return (slice_ * t.STEPS * t.A_GROUP + kg * t.BM + wm * 64 + 4 * lrow) * 4


def r_b(t, tid):
    slice_, _, wn, lrow, kg = _wave(t, tid)
    return 2 * t.A_STAGE + (slice_ * t.STEPS * t.B_GROUP + kg * t.BN + wn * 64 + 4 * lrow) * 4


STORE_2ST64 = re.compile(r"ds_write2st64_b32 %\[w([AB])\], v(\d+), v(\d+) offset0:(\d+) offset1:(\d+)$")
STORE_2 = re.compile(r"ds_write2_b32 %\[w([AB])(1?)\], v(\d+), v(\d+) offset0:(\d+) offset1:(\d+)$")
STORE_128 = re.compile(r"ds_write_b128 %\[w([AB])\], v\[(\d+):(\d+)\] offset:(\d+)$")
STORE_F = re.compile(r"ds_write_b32 %\[fst\], v(\d+) offset:(\d+)$")


def _pieces(t, tid, line):
    """(operand, [(register, byte address)]) of one store instruction
    (operand "F": the fringe variant's staged words, in the A buffer)."""
    m = STORE_F.match(line)
    if m:
        return "F", [(int(m.group(1)), f_st(t, None, tid) + int(m.group(2)))]
    m = STORE_2ST64.match(line)
    if m:
        op, r0, r1, o0, o1 = m.group(1), *(int(x) for x in m.groups()[1:])
        start = w_a(t, tid) if op == "A" else w_b(t, tid)
        return op, [(r0, start + 256 * o0), (r1, start + 256 * o1)]
    m = STORE_2.match(line)
    if m:
        op, second, r0, r1, o0, o1 = m.group(1), m.group(2), *(int(x) for x in m.groups()[2:])
        start = w_a(t, tid) if op == "A" else w_b(t, tid)
        if second:  # the second buffer's base register
            start += t.A_STAGE if op == "A" else t.B_STAGE
        return op, [(r0, start + 4 * o0), (r1, start + 4 * o1)]
    m = STORE_128.match(line)
    assert m, line
    op, r0, r3, off = m.group(1), *(int(x) for x in m.groups()[1:])
    assert r3 == r0 + 3
    start = w_a(t, tid) if op == "A" else w_b(t, tid)
    return op, [(r0 + c, start + off + 4 * c) for c in range(4)]


def _stage_stores(t, st, buf):
    """{byte address: ('A', row, k) or ('B', k, col)} written by one stage's
    stores from staging set st into buffer buf; for the fringe variant also
    ('R', k) (the extra row's element of k) and ('C', k) (the extra
    column's), which every thread of that k stores."""
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
        if t.FRINGE:
            regs[t.fa(st)] = ("R", tid % t.BK)
            regs[t.fa(st) + 1] = ("C", tid % t.BK)
        for line in lines:
            op, pieces = _pieces(t, tid, line)
            if op == "F":
                lo, hi = buf * t.A_STAGE + t.FPAD, buf * t.A_STAGE + t.FPAD + 8 * t.BK
            else:
                lo, hi = (buf * t.A_STAGE, (buf + 1) * t.A_STAGE) if op == "A" else \
                         (a_end + buf * t.B_STAGE, a_end + (buf + 1) * t.B_STAGE)
            for reg, addr in pieces:
                assert lo <= addr and addr + 4 <= hi, (t.name, tid, line)
                if op == "F":  # the same word from every thread of its k
                    assert written.get(addr, regs[reg]) == regs[reg], ("store overlap", t.name, tid, line)
                else:
                    assert addr not in written, ("store overlap", t.name, tid, line)
                    assert regs[reg][0] == op, (t.name, line)
                written[addr] = regs[reg]
    return written


@pytest.mark.parametrize("name", sorted(TILES))
@pytest.mark.parametrize("buf", [0, 1])
def test_stage_stores_follow_the_layout(name, buf):
    """Every staged element lands at its k-major word, whole stage, no
    overlap (buffer 0 is also where the C++ first stage stores: the same
    element maps and the same words)."""
    t = TILES[name]
    for st in range(t.DEPTH):
        written = _stage_stores(t, st, buf)
        assert len(written) == t.BM * t.BK + t.BK * t.BN + (2 * t.BK if t.FRINGE else 0)
        for addr, e in written.items():
            if e[0] in "RC":
                # the extra row's k at word k of the fringe words, the
                # extra column's at BK + k
                assert addr == buf * t.A_STAGE + t.FPAD + 4 * (e[1] + (t.BK if e[0] == "C" else 0)), (name, e)
                continue
            word = a_word(t, e[1], e[2]) if e[0] == "A" else b_word(t, e[1], e[2])
            shift = buf * (t.A_STAGE if e[0] == "A" else t.B_STAGE)
            assert addr == 4 * word + shift, (name, e)


@pytest.mark.parametrize("name", sorted(TILES))
@pytest.mark.parametrize("buf", [0, 1])
def test_fragment_reads_find_their_operands(name, buf):
    t = TILES[name]
    a_end = 2 * t.A_STAGE
    written = _stage_stores(t, 0, buf)
    for s in range(t.STEPS):
        lines = t.frag_reads(64, s, buf)
        offs = [int(re.search(r"offset:(\d+)", l).group(1)) for l in lines]
        for tid in range(t.THREADS):
            slice_, wm, wn, lrow, kg = _wave(t, tid)
            k = 4 * (slice_ * t.STEPS + s) + kg
            for e in range(4):
                a_addr = r_a(t, tid) + offs[0] + 4 * e
                b_addr = r_b(t, tid) + offs[1] + 4 * e
                assert 0 <= a_addr and a_addr + 4 <= a_end
                assert a_end <= b_addr and b_addr + 4 <= t.LDS
                # block e of the lane: A row 4 lrow + e, B column 4 lrow + e
                assert written[a_addr] == ("A", wm * 64 + 4 * lrow + e, k), (s, tid, e)
                assert written[b_addr] == ("B", k, wn * 64 + 4 * lrow + e), (s, tid, e)


F_READ1 = re.compile(r"ds_read_b32 v(\d+), %\[(\w+)\] offset:(\d+)$")
F_FMAC = re.compile(r"v_fmac_f32 %\[(\w+)\], v(\d+), v(\d+)$")
def f_grids(t):
    """(tiles_m, tiles_n, i, j): grids of the smallest size the variant
    takes, larger ones (4097^3's for 256 x 128), and ones whose last shares
    end inside or beyond the tile."""
    mm, mn = f_min_grid(t)
    return [(mm, mn, 0, 0), (mm, mn, mm - 1, mn - 1), (2 * mm, 2 * mn, 0, 0), (2 * mm, 2 * mn, 2 * mm - 1, 2 * mn - 1),
            (2 * mm, 2 * mn, mm - 1, mn + 1), (mm + 1, mn + 1, mm, mn), (32, 32, 31, 30), (mm + 3, mn + 3, mm + 2, mn + 2)]


FRINGE_CASES = [(n, cur, g) for n in sorted(n for n in TILES if TILES[n].FRINGE) for cur in (0, 1)
                for g in f_grids(TILES[n])]


def _fringe_products(t, grid, tid, cur, written):
    """{sum: [(element, element), ...]} the fringe FMAs of one K step on
    buffer cur compute for thread tid of the block at grid = (tiles_m,
    tiles_n, i, j), in issue order, replaying the step's fringe reads
    (registers <- the elements `written` holds at their addresses)."""
    regs, prods = {}, {}
    for line in t.k_step(cur):
        assert not line.startswith("ds_read") or "%[r" in line or F_READ1.match(line), line
        m = F_READ1.match(line)
        if m and m.group(2) in F_BASES:
            regs[int(m.group(1))] = written[F_BASES[m.group(2)](t, grid, tid) + int(m.group(3))]
            continue
        m = F_FMAC.match(line)
        if m:
            prods.setdefault(m.group(1), []).append((regs[int(m.group(2))], regs[int(m.group(3))]))
    return prods


@pytest.mark.parametrize("name,cur,grid", FRINGE_CASES, ids=[f"{n}-{c}-{g}" for n, c, g in FRINGE_CASES])
def test_fringe_sums_multiply_matching_k(name, cur, grid):
    """Per K step, thread tid adds to its row sum the extra row's k times
    B's (k, n) and to its column sum A's (m, k) times the extra column's k,
    k = tid / FP and (n, m) its share position's column and row, and to its
    corner sum the extra row's and column's k = tid % BK; so the BK sums of
    a share position, and the corner's BK, hold every k of the stage exactly
    once."""
    t = TILES[name]
    written = _stage_stores(t, 0, cur)
    for tid in range(t.THREADS):
        prods = _fringe_products(t, grid, tid, cur, written)
        k, ks = tid // t.FP, tid % t.BK
        n, m = f_cols(t, grid, tid)
        assert prods == {"frow": [(("R", k), ("B", k, n))], "fcol": [(("C", k), ("A", m, k))],
                         "fcor": [(("R", ks), ("C", ks))]}, (tid, grid)


@pytest.mark.parametrize("shape", sorted({(t.BM, t.BN) for t in G.TILES}))
def test_fringe_shares_cover_each_output_once(shape):
    """Over the blocks of a tile column the extra row's shares are
    disjoint and cover the tile's BN columns; over a tile row the extra
    column's cover its BM rows (every grid the variant takes: enough tile
    rows and columns that a share is at most FP wide); and the stored
    positions are those below the share's width."""
    t = next(x for x in G.TILES if x.FRINGE and (x.BM, x.BN) == shape)
    mm, mn = f_min_grid(t)
    for tiles_m in range(mm, 300):
        cols = []
        for i in range(tiles_m):
            cpt, _, n0, _ = f_share(t, tiles_m, mn, i, 0)
            assert cpt <= t.FP
            cols += [n0 + c for c in range(t.FP) if c < cpt and n0 + c < t.BN]
        assert sorted(cols) == list(range(t.BN)), tiles_m
    for tiles_n in range(mn, 600):
        rows = []
        for j in range(tiles_n):
            _, rpt, _, m0 = f_share(t, mm, tiles_n, 0, j)
            assert rpt <= t.FP
            rows += [m0 + c for c in range(t.FP) if c < rpt and m0 + c < t.BM]
        assert sorted(rows) == list(range(t.BM)), tiles_n


@pytest.mark.parametrize("name", sorted(TILES))
def test_k_slices_cover_every_step_once(name):
    """The wavefronts that share a wave tile take disjoint runs of a stage's
    MFMA steps that together cover all of them."""
    t = TILES[name]
    steps = sorted(sl * t.STEPS + s for sl in range(t.KSLICES) for s in range(t.STEPS))
    assert steps == list(range(t.GROUPS))


def _bank_conflict_free_32bit(addrs):
    """The 32 words of one half-wavefront's 32-bit write lie in 32 different
    banks.  A 32-bit store is served per half-wavefront and words 32 apart
    share a bank there (bank = word mod 32): the level-6 kernel's
    transposing store measured bank-conflict cycles with rows 136 words
    apart (its two k-groups 544 words, 32 mod 64, apart) and none at 132
    (16 apart), and this loop's 64 x 64 tile measured 1.40 conflict cycles
    per LDS instruction with half-wavefronts of 2 rows x 16 four-k groups
    260 words apart."""
    return len({(a // 4) % 32 for a in addrs}) == len(addrs)


@pytest.mark.parametrize("name", sorted(TILES))
def test_transposing_stores_hit_distinct_banks(name):
    """Each half-wavefront of a 32-bit transposing store writes 32 different
    banks (the padded groups' purpose)."""
    t = TILES[name]
    for line in t.stage_stores(0, 0):
        if line.startswith(("ds_write_b128", "ds_write_b32 %[fst]")):
            continue
        for first in range(0, t.THREADS, 32):
            for piece in (0, 1):
                addrs = [_pieces(t, tid, line)[1][piece][1] for tid in range(first, first + 32)]
                assert _bank_conflict_free_32bit(addrs), (name, line, first, piece)


@pytest.mark.parametrize("name", sorted(TILES))
def test_whole_stores_and_fragment_reads_hit_distinct_banks(name):
    """128-bit stores and reads: each group of 16 lanes (one pass of 64
    words) covers 64 different banks (bank = word mod 64)."""
    t = TILES[name]
    lines = [l for l in t.stage_stores(0, 0) if l.startswith("ds_write_b128")]
    for line in lines:
        for first in range(0, t.THREADS, 16):
            words = [(_pieces(t, tid, line)[1][0][1] // 4 + c) % 64
                     for tid in range(first, first + 16) for c in range(4)]
            assert len(set(words)) == 64, (name, line, first)
    for s in range(t.STEPS):
        offs = [int(re.search(r"offset:(\d+)", l).group(1)) for l in t.frag_reads(64, s, 0)]
        for first in range(0, t.THREADS, 16):
            for r, off in ((r_a, offs[0]), (r_b, offs[1])):
                words = [((r(t, tid) + off) // 4 + c) % 64 for tid in range(first, first + 16) for c in range(4)]
                assert len(set(words)) == 64, (name, s, first)


@pytest.mark.parametrize("name", sorted(TILES))
def test_loop_structure(name):
    t = TILES[name]
    prog = t.program()
    mfmas = [l for l in prog if l.startswith("v_mfma")]
    # the prologue issues no MFMA; a pair of K steps and the odd step, each
    # STEPS MFMA steps of 16
    assert len(mfmas) == 3 * 16 * t.STEPS
    # every accumulator block gets one MFMA per step
    for b in range(16):
        assert sum(1 for l in mfmas if l.startswith(f"v_mfma_f32_16x16x4_f32 v[{4*b}:")) == 3 * t.STEPS
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
    per_stage = t.LOADS
    for cur in (0, 1):
        step = t.k_step(cur)
        first_store = next(i for i, l in enumerate(step) if l.startswith("ds_write"))
        waits = [l for l in step[:first_store] if l.startswith("s_waitcnt vmcnt")]
        assert waits == [f"s_waitcnt vmcnt({per_stage * (t.DEPTH - 1)})"]
        last_store = max(i for i, l in enumerate(step) if l.startswith("ds_write"))
        first_load = next(i for i, l in enumerate(step) if l.startswith("buffer_load"))
        assert "s_waitcnt lgkmcnt(0)" in step[last_store:first_load]


# -- the loop's waits, modelled ------------------------------------------------
# LDS instructions complete in the order they are issued, and so do the
# buffer loads (the loop issues no scalar memory load, which would complete
# out of order); s_waitcnt lgkmcnt(N) / vmcnt(N) returns once at most the
# youngest N are outstanding.
_VREGS = re.compile(r"\bv\[(\d+):(\d+)\]|\bv(\d+)\b")


def _regs(text):
    out = set()
    for lo, hi, one in _VREGS.findall(text):
        out |= set(range(int(lo), int(hi) + 1)) if lo else {int(one)}
    return out


def check_waits(lines, in_flight_loads=(), in_flight_stores=1):
    """Replay the waits of a straight-line run of the loop: every MFMA
    operand (and fringe FMA operand) has arrived from its LDS read, every
    stage store reads a
    staging register whose load has arrived, no staging register is
    reloaded while a store still reads it, and no LDS access is outstanding
    at a barrier.  The run starts with the prelude's loads and the C++
    part's stage-0 stores (registers the loop does not name) in flight.
    Returns the list of violations."""
    lds = [("w", set())] * in_flight_stores   # outstanding LDS ops: ("r", regs written) / ("w", regs read)
    vm = list(in_flight_loads)     # outstanding buffer loads: regs written
    bad = []
    for i, line in enumerate(lines):
        if line.startswith("s_waitcnt"):
            m = re.search(r"lgkmcnt\((\d+)\)", line)
            if m:
                keep = int(m.group(1))
                lds = lds[len(lds) - keep:] if keep else []
            m = re.search(r"vmcnt\((\d+)\)", line)
            if m:
                keep = int(m.group(1))
                vm = vm[len(vm) - keep:] if keep else []
        elif line.startswith("ds_read"):
            lds.append(("r", _regs(line.split(",")[0])))
        elif line.startswith("ds_write"):
            srcs = _regs(line.split(",", 1)[1])
            if any(srcs & regs for regs in vm):
                bad.append((i, line, "stores a register whose load is outstanding"))
            lds.append(("w", srcs))
        elif line.startswith("buffer_load"):
            dst = _regs(line.split(",")[0])
            if any(kind == "w" and dst & regs for kind, regs in lds):
                bad.append((i, line, "reloads a register an outstanding store reads"))
            vm.append(dst)
        elif line.startswith("v_mfma"):
            ops = _regs(line.split(",", 1)[1].rsplit(",", 1)[0])
            if any(kind == "r" and ops & regs for kind, regs in lds):
                bad.append((i, line, "reads a fragment whose LDS read is outstanding"))
        elif line.startswith("v_fmac"):
            ops = _regs(line.split(",", 1)[1])
            if any(kind == "r" and ops & regs for kind, regs in lds):
                bad.append((i, line, "multiplies a word whose LDS read is outstanding"))
        elif line == "s_barrier":
            if lds:
                bad.append((i, line, "LDS accesses outstanding at the barrier"))
    return bad


def _steady_state(t):
    prologue = t.program()[:t.program().index("s_cmp_eq_u32 %[pairs], 0")]
    loads = [_regs(l.split(",")[0]) for l in t.prelude() if l.startswith("buffer_load")]
    return prologue + t.k_step(0) + t.k_step(1) + t.k_step(0) + t.k_step(1), loads


@pytest.mark.parametrize("name", sorted(TILES))
def test_waits_cover_every_use(name):
    t = TILES[name]
    lines, loads = _steady_state(t)
    assert check_waits(lines, loads) == []


@pytest.mark.parametrize("name", sorted(TILES))
def test_wait_model_catches_a_short_wait(name):
    """Each wait is needed: loosening any lgkmcnt / vmcnt of the loop by
    one is reported -- except an lgkmcnt held at the field's top (15),
    which already waits for more than it needs."""
    t = TILES[name]
    lines, loads = _steady_state(t)
    waits = [i for i, l in enumerate(lines) if l.startswith("s_waitcnt") and "lgkmcnt(15)" not in l]
    for i in waits:
        loose = re.sub(r"(lgkmcnt|vmcnt)\((\d+)\)", lambda m: f"{m.group(1)}({int(m.group(2)) + 1})", lines[i])
        assert check_waits(lines[:i] + [loose] + lines[i + 1:], loads), (name, i, lines[i])


@pytest.mark.parametrize("name", sorted(TILES))
def test_wait_counts_fit_their_fields(name):
    """gfx9 encodes lgkmcnt in 4 bits and vmcnt in 6."""
    for line in TILES[name].program() + TILES[name].prelude():
        for field, top in (("lgkmcnt", 15), ("vmcnt", 63)):
            m = re.search(field + r"\((\d+)\)", line)
            assert m is None or int(m.group(1)) <= top, line
