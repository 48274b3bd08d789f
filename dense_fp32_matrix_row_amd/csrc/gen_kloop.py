"""Write l10_kloop.inc: the K loops of level 10's whole-tile kernels
(l10_kloop.hip) as GCN assembly text for gfx950.

The kernels' C++ part sets up addresses, stores the first stage and runs
the epilogue; each loop is emitted instruction by instruction so that the
order of the matrix, LDS and global-memory instructions is the one chosen
here rather than the compiler's.  [CP04] (section on boundary conditions
and limits, the gap analysis against cuBLAS) puts the last 15-20 % of an
FP32 GEMM in exactly this instruction-level ordering, out of reach of C++;
its double-buffering section gives the overlap these loops implement.

Two tiles, both of 64 x 64 wavefront tiles (4 x 4 blocks of
v_mfma_f32_16x16x4_f32) over a 128-column block tile with 16-deep stages,
each in the four operand orientations (only the stage loads and stores
differ: a row-major A and a transposed B are transposed into LDS, a
transposed A and a row-major B are stored whole):
  256 x 128, eight wavefronts (4 x 2), two blocks per CU: one stage of
            global prefetch (the other block's wavefronts cover the wait);
  128 x 128, four wavefronts (2 x 2), one wavefront per SIMD where one
            block runs per CU: two stages of global prefetch in two
            register sets.

Each tile also has a fringe variant, for a grid with one more row of C
below it and / or one more column to its right (M = BM a + 1, N = BN b + 1):
every block holds, over its K loop, all of A for its BM rows and all of B
for its BN columns, so it can also sum the extra row of A against a share
of its columns and a share of its rows against the extra column of B (at
most THREADS / BK of each per block, so that each block adds only a few
vector-ALU FMAs per stage: 8 and 8 at 4097^3 on 256 x 128), and the one
corner element.  The BK values of the extra row and column per stage travel
like the stage itself (loaded with it, stored after it into 2 BK words
after the A stage), so that nothing of A or B is read a second time.

Stage 0 is the first K % 16 k (a whole stage when K % 16 == 0), zero-padded,
and is put into LDS buffer 0 by the kernel's C++ part; every stage the
assembly loads (from stage 1 on, at that offset) is whole.  Each tile has
two statements: a prelude that requests stages 1 .. DEPTH, issued before the
C++ part's stage-0 loads so that the latencies overlap, and the loop.

Register map (the kernels pin these with asm operand constraints/clobbers):
  s[60:63], s[64:67]  buffer resources of A and B, based at the next stage
            to load, record counts ending at the tile's last element
  v[0:63]   accumulators: 16 blocks of 16 x 16 (block b = 4 i + j at
            v[4b : 4b+3], i = A block, j = B block)
  v[64:71]  fragment set E: A operands of blocks i = 0..3 (v64..v67) and B
            operands of blocks j = 0..3 (v68..v71) for one MFMA step
  v[72:79]  fragment set O, the same for the alternate step
  v[80:..]  global-load staging: per set, the A float4s then the B float4s
            of one stage (12 words for 256 x 128, 16 for 128 x 128)
  fringe variant: after the staging sets, one register pair per set
            stages the extra row's and column's value of the thread's k
            (tid % BK) like the stage (v92 / v93 for 256 x 128); the next
            six hold the LDS words the fringe FMAs read; its three sums
            (row, column, corner) are compiler-placed operands

One K step (16 deep) per wavefront: four MFMA steps s = 0..3 of 16 MFMAs,
step s reading k = 4 s + lane / 16.  Step s runs on one fragment set while
the other set receives step s + 1 (128-bit LDS reads issued after the
step's first MFMA); the next stage is stored from its staging set into the
free LDS buffer during step 0 and the same set is reloaded (with the stage
one or two further on) during step 1 -- for the tiles with two staging sets,
the stores spread over steps 0 and 1 and the reload waits for step 2; the
barrier sits halfway through
step 3, after which step 0 of the next stage is read from the other buffer,
so the LDS latency after a barrier hides under the remaining eight MFMAs.
Loop bookkeeping is scalar (buffer resources advanced in SGPRs, LDS offsets
immediate), so the loop issues no vector-ALU instruction besides the MFMAs.

Run as a script to rewrite l10_kloop.inc; tests check that the committed
file equals what this script emits.
"""

from __future__ import annotations

import os

FE, FO = 64, 72                # fragment sets
STAGING = 80                   # first staging register
RES_A, RES_B = 60, 64          # buffer resources of A and B: s[60:63], s[64:67]

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "l10_kloop.inc")


def _round256(n: int) -> int:
    return -(-n // 256) * 256


class Tile:
    """One block tile of BM x BN, 64 x 64 wavefront tiles (WAVES_M x WAVES_N
    of them, each shared by KSLICES wavefronts that split every stage's MFMA
    steps), BK-deep stages, DEPTH staging register sets, operands as stored
    (TA: A given transposed, K x M; TB: B given transposed, N x K)."""

    def __init__(self, bm: int, bn: int, bk: int, waves_m: int, waves_n: int, kslices: int,
                 depth: int, ta: bool = False, tb: bool = False, fringe: bool = False):
        self.BM, self.BN, self.BK = bm, bn, bk
        self.WAVES_M, self.WAVES_N, self.KSLICES, self.DEPTH = waves_m, waves_n, kslices, depth
        self.TA, self.TB, self.FRINGE = ta, tb, fringe
        self.THREADS = 64 * waves_m * waves_n * kslices
        self.GROUPS = bk // 4                         # four-k groups (MFMA steps) per stage
        self.STEPS = self.GROUPS // kslices           # MFMA steps per stage per wavefront
        # floats per four-k group: a few words of pad where the stage store
        # transposes (a row-major A, a transposed B), so that its 32-bit
        # writes hit 32 different banks per half-wavefront (words 32 apart
        # share a bank there; with the 64-deep stage's pad of 4 that also
        # takes the kernel's lane order of 4 majors x 8 groups per
        # half-wavefront)
        pad = 8 if bk == 16 else 4
        self.A_GROUP = 4 * bm + (0 if ta else pad)
        self.B_GROUP = 4 * bn + (pad if tb else 0)
        # bytes per stage, a whole number of 256; the fringe variant's words
        # (BK of the extra row, then BK of the extra column) at FPAD after
        # the groups
        self.FPAD = self.GROUPS * self.A_GROUP * 4
        self.A_STAGE = _round256(self.FPAD + (8 * bk if fringe else 0))
        self.B_STAGE = _round256(self.GROUPS * self.B_GROUP * 4)
        self.A_LOADS = bm * bk // 4 // self.THREADS   # A float4s per thread per stage
        self.B_LOADS = bk * bn // 4 // self.THREADS   # B float4s per thread per stage
        self.SET = 4 * (self.A_LOADS + self.B_LOADS)  # staging words per set
        # buffer loads per stage (the fringe variant: one word of the extra
        # row and one of the extra column per thread)
        self.LOADS = self.A_LOADS + self.B_LOADS + (2 if fringe else 0)
        # fringe variant: positions of its share per k (thread tid takes k =
        # tid / FP, position tid % FP), registers after the staging sets
        self.FP = self.THREADS // bk
        self.F_STAGE = STAGING + depth * self.SET
        self.FT = self.F_STAGE + 2 * depth
        self.LDS = 2 * self.A_STAGE + 2 * self.B_STAGE
        assert bm == 64 * waves_m and bn == 64 * waves_n and self.STEPS >= 2
        assert self.A_LOADS * self.THREADS * 4 == bm * bk and self.B_LOADS * self.THREADS * 4 == bk * bn
        assert self.last_vgpr() < 256 and self.THREADS % bk == 0

    @property
    def name(self) -> str:
        return f"{self.BM}x{self.BN}_{'T' if self.TA else 'N'}{'T' if self.TB else 'N'}" + \
            ("_F" if self.FRINGE else "")

    def last_vgpr(self) -> int:
        return self.FT + 5 if self.FRINGE else STAGING + self.DEPTH * self.SET - 1

    def last_staging(self) -> int:
        """Last register a load of the prelude leaves in flight."""
        return self.FT - 1 if self.FRINGE else STAGING + self.DEPTH * self.SET - 1

    def fa(self, st: int) -> int:
        """Fringe variant: staging register of the extra row's word (set st);
        the extra column's is the next."""
        return self.F_STAGE + 2 * st

    # -- per-thread element maps (restated by the kernel and the tests) ------
    def a_per(self) -> int:
        """A float4s per row (row-major A) or per k-row (transposed A)."""
        return self.BM // 4 if self.TA else self.BK // 4

    def b_per(self) -> int:
        return self.BK // 4 if self.TB else self.BN // 4

    # -- instruction builders ------------------------------------------------
    def mfma(self, b: int, fs: int) -> str:
        i, j = divmod(b, 4)
        return f"v_mfma_f32_16x16x4_f32 v[{4*b}:{4*b+3}], v{fs+i}, v{fs+4+j}, v[{4*b}:{4*b+3}]"

    def frag_reads(self, fs: int, s: int, buf: int) -> list[str]:
        """MFMA step s (of this wavefront's slice) of LDS buffer buf into
        fragment set fs; the kernel's base addresses point at the slice's
        first group."""
        return [f"ds_read_b128 v[{fs}:{fs+3}], %[rA] offset:{s * self.A_GROUP * 4 + buf * self.A_STAGE}",
                f"ds_read_b128 v[{fs+4}:{fs+7}], %[rB] offset:{s * self.B_GROUP * 4 + buf * self.B_STAGE}"]

    def set_base(self, st: int) -> int:
        return STAGING + st * self.SET

    def loads(self, st: int) -> list[str]:
        """One stage into staging set st: A float4s first, then B float4s
        (which elements each thread loads is set by the kernel's per-thread
        offsets; see stage_stores)."""
        r = self.set_base(st)
        out = [f"buffer_load_dwordx4 v[{r + 4*h}:{r + 4*h + 3}], %[oA{h}], s[{RES_A}:{RES_A + 3}], 0 offen"
               for h in range(self.A_LOADS)]
        rb = r + 4 * self.A_LOADS
        out += [f"buffer_load_dwordx4 v[{rb + 4*h}:{rb + 4*h + 3}], %[oB{h}], s[{RES_B}:{RES_B + 3}], 0 offen"
                for h in range(self.B_LOADS)]
        if self.FRINGE:
            # the extra row's element of k and the extra column's, same
            # stage, k = tid % BK, through the same resources
            out += [f"buffer_load_dword v{self.fa(st)}, %[foa], s[{RES_A}:{RES_A + 3}], 0 offen",
                    f"buffer_load_dword v{self.fa(st) + 1}, %[fob], s[{RES_B}:{RES_B + 3}], 0 offen"]
        return out

    # The next stage of each operand: the resource's base moves one stage on
    # (48-bit address: carry into the high word) and its record count drops
    # by as much, stopping at 0.  The loads carry no scalar offset, so the
    # range check, which covers the per-thread offset, bounds every load by
    # the operand's last element whatever the hardware does with a scalar
    # offset: a stage loaded past K reads zeros without touching memory.
    ADVANCE = [f"s_add_u32 s{RES_A}, s{RES_A}, %[stepA]", f"s_addc_u32 s{RES_A + 1}, s{RES_A + 1}, 0",
               f"s_sub_u32 s{RES_A + 2}, s{RES_A + 2}, %[stepA]", f"s_cselect_b32 s{RES_A + 2}, 0, s{RES_A + 2}",
               f"s_add_u32 s{RES_B}, s{RES_B}, %[stepB]", f"s_addc_u32 s{RES_B + 1}, s{RES_B + 1}, 0",
               f"s_sub_u32 s{RES_B + 2}, s{RES_B + 2}, %[stepB]", f"s_cselect_b32 s{RES_B + 2}, 0, s{RES_B + 2}"]

    @staticmethod
    def _transposing(w: str, r: int, buf: int, stage: int, row: int, copy: int, copies: int) -> list[str]:
        """Float4s v[r + 4h ..] that each hold k = 4 q .. 4 q + 3 of one m
        (n) go to four k-rows of group q, `row` words apart; copy h is
        h `copy` words further.  Offsets in 256-byte units where every one
        is a whole number of them (ds_write2st64_b32, the buffer as an
        offset), else in words (ds_write2_b32, the buffer by its own base
        register)."""
        out = []
        if row % 64 == 0 and copy % 64 == 0:
            u = buf * (stage // 256)
            for h in range(copies):
                for c0, c1 in ((0, 1), (2, 3)):
                    out.append(f"ds_write2st64_b32 %[{w}], v{r + 4*h + c0}, v{r + 4*h + c1} "
                               f"offset0:{u + (c0 * row + h * copy) // 64} "
                               f"offset1:{u + (c1 * row + h * copy) // 64}")
        else:
            base = w if buf == 0 else w + "1"
            for h in range(copies):
                for c0, c1 in ((0, 1), (2, 3)):
                    o0, o1 = c0 * row + h * copy, c1 * row + h * copy
                    assert o1 <= 255
                    out.append(f"ds_write2_b32 %[{base}], v{r + 4*h + c0}, v{r + 4*h + c1} "
                               f"offset0:{o0} offset1:{o1}")
        return out

    def stage_stores(self, st: int, buf: int) -> list[str]:
        """Staging set st into LDS buffer buf.  Element maps (copy h of
        thread tid; per = float4s per row or k-row, a_per / b_per; (j, q)
        the thread's slot, (tid/per, tid%per) except for a transposing
        store with per 16, whose half-wavefronts take 4 majors x 8 groups):
          A row-major:  row j + h THREADS/per, k 4 q .. +3:
                        transposed into four k-rows of a group;
          A transposed: k-row j + h THREADS/per, rows 4 q ..:
                        stored whole;
          B row-major:  k-row j + h THREADS/per, columns 4 q ..:
                        stored whole;
          B transposed: column j + h THREADS/per, k 4 q .. +3:
                        transposed.
        Only the per-thread bases differ between the slot orders; the
        offsets here (h THREADS/per majors, c k-rows) are the same."""
        r = self.set_base(st)
        rb = r + 4 * self.A_LOADS
        out = []
        if self.TA:
            dk = self.THREADS // self.a_per()
            assert dk % 4 == 0
            for h in range(self.A_LOADS):
                out.append(f"ds_write_b128 %[wA], v[{r + 4*h}:{r + 4*h + 3}] "
                           f"offset:{buf * self.A_STAGE + h * (dk // 4) * self.A_GROUP * 4}")
        else:
            out += self._transposing("wA", r, buf, self.A_STAGE, self.BM,
                                     self.THREADS // self.a_per(), self.A_LOADS)
        if self.TB:
            out += self._transposing("wB", rb, buf, self.B_STAGE, self.BN,
                                     self.THREADS // self.b_per(), self.B_LOADS)
        else:
            dk = self.THREADS // self.b_per()
            assert dk % 4 == 0
            for h in range(self.B_LOADS):
                out.append(f"ds_write_b128 %[wB], v[{rb + 4*h}:{rb + 4*h + 3}] "
                           f"offset:{buf * self.B_STAGE + h * (dk // 4) * self.B_GROUP * 4}")
        if self.FRINGE:
            # word k of the extra row, word BK + k of the extra column
            # (%[fst] = 4 (tid % BK); the THREADS / BK threads of each k store
            # the same value)
            pad = buf * self.A_STAGE + self.FPAD
            out += [f"ds_write_b32 %[fst], v{self.fa(st)} offset:{pad}",
                    f"ds_write_b32 %[fst], v{self.fa(st) + 1} offset:{pad + 4 * self.BK}"]
        return out

    def fringe_reads(self, cur: int) -> list[str]:
        """The fringe variant's LDS reads of one stage on buffer cur.  Per
        thread, with k = tid / FP of the stage:
          row sum (%[frow]): B's word (k, n) of one of the block's columns
            (%[frB]) times the extra row's word k (%[fpk]);
          column sum (%[fcol]): A's word (m, k) of one of the block's rows
            (%[fcA]) times the extra column's word k (%[fpk], 4 BK bytes on);
          corner (%[fcor]): the extra row's and column's words of
            k = tid % BK (%[fst]).
        The kernel sets which column and row (n, m) a thread takes."""
        a0 = cur * self.A_STAGE
        pad = a0 + self.FPAD
        col = 4 * self.BK
        t = [f"v{self.FT + i}" for i in range(6)]
        return [f"ds_read_b32 {t[0]}, %[frB] offset:{cur * self.B_STAGE}",
                f"ds_read_b32 {t[1]}, %[fpk] offset:{pad}",
                f"ds_read_b32 {t[2]}, %[fcA] offset:{a0}",
                f"ds_read_b32 {t[3]}, %[fpk] offset:{pad + col}",
                f"ds_read_b32 {t[4]}, %[fst] offset:{pad}",
                f"ds_read_b32 {t[5]}, %[fst] offset:{pad + col}"]

    def fringe_fmas(self) -> list[str]:
        t = [f"v{self.FT + i}" for i in range(6)]
        return [f"v_fmac_f32 %[frow], {t[1]}, {t[0]}", f"v_fmac_f32 %[fcol], {t[3]}, {t[2]}",
                f"v_fmac_f32 %[fcor], {t[4]}, {t[5]}"]

    # -- the loop ------------------------------------------------------------
    def k_step(self, cur: int) -> list[str]:
        """One K step (stage) on LDS buffer cur (stage n with n % 2 == cur);
        on entry set E is being read with this wavefront's first MFMA step
        of stage n and stage n + 1 is in flight in staging set
        (n + 1) % DEPTH (with DEPTH 2, stage n + 2 in the other set behind
        it)."""
        nxt = 1 - cur
        st = nxt % self.DEPTH
        per_stage = self.LOADS
        sets = (FE, FO)
        stores = self.stage_stores(st, nxt)
        loads = self.loads(st)
        assert len(loads) + 1 < 16
        # stores after MFMAs 1..12 of the first step (spread when more than
        # 12), so that the last one has three MFMAs to complete in before the
        # next step's lgkmcnt(0): with one wavefront per SIMD nothing else
        # would cover that wait (measured: 1024 x 1024 x 4096 on the 64 x 64
        # tile 122 -> 125 TFLOP/s against stores after MFMAs 4..15)
        # With two staging sets (a stage loaded two ahead), the stores spread
        # over steps 0 and 1 and the set is reloaded in step 2: a burst of
        # the whole stage's stores in step 0, from every wavefront of the
        # CU at once, fills the LDS data queue and delays the fragment reads
        # queued behind it (1024 x 1024 x 8192 on the 64 x 64 tile: 23x the
        # vendor kernel's SQ_LDS_DATA_FIFO_FULL).  Step 1 then waits only
        # for its fragment reads: LDS accesses complete in issue order, and
        # the reads precede step 0's stores, so lgkmcnt(<stores in step 0>)
        # suffices (lgkmcnt is a 4-bit field).
        spread = self.DEPTH >= 2
        span = 28 if spread else 12          # MFMA slots the stores occupy
        store_at: dict[tuple[int, int], list[str]] = {}
        for i, ins in enumerate(stores):
            slot = 1 + i if len(stores) <= 12 and not spread else 1 + i * span // len(stores)
            store_at.setdefault(divmod(slot, 16), []).append(ins)
        in_step0 = sum(len(v) for (st_, _), v in store_at.items() if st_ == 0)
        reload_step = 2 if spread else 1
        out = []
        for ss in range(self.STEPS):
            fs, fn = sets[ss % 2], sets[(ss + 1) % 2]
            mf = [self.mfma(b, fs) for b in range(16)]
            # work placed after MFMA i of this step
            extra: dict[int, list[str]] = {}
            if ss == 0:
                # stage n + 1 complete (its set's loads are the older ones in
                # flight), then stored into the free buffer
                extra.setdefault(0, []).append(f"s_waitcnt vmcnt({per_stage * (self.DEPTH - 1)})")
            for (st_, slot), ins in store_at.items():
                if st_ == ss:
                    extra.setdefault(slot, []).extend(ins)
            if ss == reload_step:
                # the stores have completed (lgkmcnt(0) at this step's start),
                # so the staging set may take stage n + 1 + DEPTH
                for i, ins in enumerate(loads):
                    extra.setdefault(1 + i, []).append(ins)
                extra.setdefault(len(loads) + 1, []).extend(self.ADVANCE)
            if self.FRINGE:
                # the fringe's reads of this stage and, a step later, its
                # FMAs.  With one staging set: reads after MFMA 6 of the first
                # step, FMAs after MFMA 2 of the second (the other wavefronts
                # of the SIMD keep the matrix pipe busy).  With two: reads
                # two per slot after the second step's stores (slots 13-15),
                # FMAs one per slot after the third step's loads (12-14), so
                # that a wavefront alone on its SIMD issues few of them
                # between two MFMAs; either way they complete at the next
                # step's lgkmcnt(0), before the last step's barrier.
                reads, fmas = self.fringe_reads(cur), self.fringe_fmas()
                if not spread and ss == 0:
                    extra.setdefault(6, []).extend(reads)
                if not spread and ss == 1:
                    extra.setdefault(2, []).extend(fmas)
                if spread and ss == 1:
                    for i, ins in enumerate(reads):
                        extra.setdefault(13 + i // 2, []).append(ins)
                if spread and ss == 2:
                    for i, ins in enumerate(fmas):
                        extra.setdefault(12 + i, []).append(ins)
            out.append(f"s_waitcnt lgkmcnt({min(in_step0, 15)})" if spread and ss == 1
                       else "s_waitcnt lgkmcnt(0)")
            last = ss == self.STEPS - 1
            for b in range(16):
                if last and b == 8:
                    # every wavefront's reads of this buffer and stores of the
                    # next are complete here (lgkmcnt(0) at the step's start)
                    out += ["s_barrier", *self.frag_reads(fn, 0, nxt)]
                out.append(mf[b])
                if not last and b == 0:
                    out += self.frag_reads(fn, ss + 1, cur)
                out += extra.get(b, [])
        return out

    def prelude(self) -> list[str]:
        """The first statement: stages 1 .. DEPTH requested into staging sets
        1 % DEPTH .., before the kernel's C++ part loads stage 0, so that
        their memory latencies overlap (one round trip before the loop
        instead of two).  The compiler cannot see into the statement, so the
        wait states a buffer load needs after a vector-ALU write of its
        descriptor or offset SGPRs (5 on gfx9) come first, whatever precedes
        it.  The loads are still in flight when the statement ends: the
        staging registers are its outputs, and the loop statement's inputs,
        pinned to the same registers."""
        out = ["s_nop 4"]
        for j in range(1, self.DEPTH + 1):
            out += [*self.loads(j % self.DEPTH), *self.ADVANCE]
        return out

    def program(self) -> list[str]:
        # stage 0 was stored into buffer 0 by the kernel's C++ part between
        # the prelude and this statement; its stores complete, then the
        # barrier makes every wavefront's visible
        prologue = ["s_waitcnt lgkmcnt(0)", "s_barrier", *self.frag_reads(FE, 0, 0)]
        pairs = ["s_cmp_eq_u32 %[pairs], 0", "s_cbranch_scc1 .Lkloop_odd_%=", ".Lkloop_pair_%=:",
                 *self.k_step(0), *self.k_step(1),
                 "s_sub_u32 %[pairs], %[pairs], 1", "s_cmp_lg_u32 %[pairs], 0",
                 "s_cbranch_scc1 .Lkloop_pair_%="]
        odd = [".Lkloop_odd_%=:", "s_cmp_eq_u32 %[odd], 0", "s_cbranch_scc1 .Lkloop_end_%=",
               *self.k_step(0), ".Lkloop_end_%=:"]
        # drain every load (the staging and fragment registers are free after
        # the asm statement) and give the last MFMAs' results the wait states
        # a vector read of them needs
        tail = ["s_waitcnt vmcnt(0) lgkmcnt(0)", "s_nop 7", "s_nop 7"]
        return prologue + pairs + odd + tail


# (BM, BN, BK, WAVES_M, WAVES_N, KSLICES, DEPTH)
SHAPES = [(256, 128, 16, 4, 2, 1, 1), (128, 128, 16, 2, 2, 1, 2), (64, 64, 64, 1, 1, 4, 2)]
TILES = [Tile(*shape, ta, tb) for shape in SHAPES for ta in (False, True) for tb in (False, True)]
TILES += [Tile(*shape, ta, tb, fringe=True) for shape in SHAPES for ta in (False, True) for tb in (False, True)]


def render() -> str:
    lines = ["// Generated by gen_kloop.py (the K loops of l10_kloop.hip); do not edit."]
    for t in TILES:
        for macro, prog in (("PRE", t.prelude()), ("ASM", t.program())):
            lines.append(f"#define SGEMM_KLOOP_{macro}_{t.name} \\")
            lines += [f'  "{ins}\\n" \\' for ins in prog]
            lines.append('  ""')
        # staging registers: outputs of the prelude (written by loads still
        # in flight, so early-clobber: no input may share them), then
        # read-write operands of the loop; the fragment sets are clobbers
        # (the fringe variant: also its two staged values, and its sums as
        # read-write operands of the loop; its LDS words are clobbers)
        quads = range(t.DEPTH * t.SET // 4)
        out = ", ".join(f'"=&{{v[{STAGING + 4*q}:{STAGING + 4*q + 3}]}}"(stg[{q}])' for q in quads)
        io = ", ".join(f'"+{{v[{STAGING + 4*q}:{STAGING + 4*q + 3}]}}"(stg[{q}])' for q in quads)
        clobbered = list(range(FE, STAGING))
        if t.FRINGE:
            for st in range(t.DEPTH):
                out += f', "=&{{v{t.fa(st)}}}"(fa[{st}]), "=&{{v{t.fa(st) + 1}}}"(fb[{st}])'
                io += f', "+{{v{t.fa(st)}}}"(fa[{st}]), "+{{v{t.fa(st) + 1}}}"(fb[{st}])'
            io += ', [frow] "+v"(frow), [fcol] "+v"(fcol), [fcor] "+v"(fcor)'
            clobbered += list(range(t.FT, t.FT + 6))
        lines.append(f"#define SGEMM_KLOOP_STAGING_OUT_{t.name} {out}")
        lines.append(f"#define SGEMM_KLOOP_STAGING_IO_{t.name} {io}")
        regs = ", ".join(f'"v{r}"' for r in clobbered)
        lines.append(f"#define SGEMM_KLOOP_CLOBBERS_{t.name} {regs}")
    return "\n".join(lines) + "\n"


if __name__ == "__main__":
    with open(OUT, "w") as f:
        f.write(render())
    print(OUT)
