"""Write l10_kloop.inc: the K loop of the 256 x 128 whole-tile kernel
(l10_kloop.hip) as GCN assembly text for gfx950.

The kernel's C++ part sets up addresses and runs the epilogue; this loop is
emitted instruction by instruction so that the order of the matrix, LDS and
global-memory instructions is the one chosen here rather than the
compiler's.  [CP04] (section on boundary conditions and limits, the gap
analysis against cuBLAS) puts the last 15-20 % of an FP32 GEMM in exactly
this instruction-level ordering, out of reach of C++; its double-buffering
section gives the overlap this loop implements.

Stage 0 is the first K % 16 k (a whole stage when K % 16 == 0), zero-padded,
and is put into LDS buffer 0 by the kernel's C++ part; the loop starts by
loading stage 1 at that offset, so every stage it loads is whole.

Register map (the kernel pins these with asm operand constraints/clobbers):
  v[0:63]   accumulators: 16 blocks of 16 x 16 (block b = 4 i + j at
            v[4b : 4b+3], i = A block, j = B block)
  v[64:71]  fragment set E: A operands of blocks i = 0..3 (v64..v67) and B
            operands of blocks j = 0..3 (v68..v71) for one MFMA step
  v[72:79]  fragment set O, the same for the alternate step
  v[80:91]  the next stage's global loads (two A float4s, one B float4)

One K step (16 deep) per wavefront: four MFMA steps s = 0..3 of 16
v_mfma_f32_16x16x4_f32 each, step s reading k = 4 s + lane / 16.  Step s
runs on one fragment set while the other set receives step s + 1 (128-bit
LDS reads issued after the step's first MFMA); the stage after next is
stored into the free LDS buffer during step 0 and its successor's global
loads go out during step 1; the barrier sits halfway through step 3, after
which step 0 of the next stage is read from the other buffer, so the LDS
latency after a barrier hides under the remaining eight MFMAs.  Loop
bookkeeping is scalar (buffer offsets in SGPRs, LDS offsets immediate), so
the loop issues no vector-ALU instruction besides the MFMAs.

Run as a script to rewrite l10_kloop.inc; tests check that the committed
file equals what this script emits.
"""

from __future__ import annotations

import os

BM, BN, BK = 256, 128, 16
A_GROUP = 4 * BM + 8           # floats per four-k group of an A stage (8 words of pad)
A_STAGE = 16640                # bytes per A stage: 4 groups, rounded up to 65 * 256
B_STAGE = BK * BN * 4          # bytes per B stage
assert 4 * A_GROUP * 4 <= A_STAGE and A_STAGE % 256 == 0
FE, FO = 64, 72                # fragment sets

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "l10_kloop.inc")


def mfma(b: int, fs: int) -> str:
    i, j = divmod(b, 4)
    return f"v_mfma_f32_16x16x4_f32 v[{4*b}:{4*b+3}], v{fs+i}, v{fs+4+j}, v[{4*b}:{4*b+3}]"


def frag_reads(fs: int, s: int, buf: int) -> list[str]:
    """MFMA step s of LDS buffer buf into fragment set fs."""
    return [f"ds_read_b128 v[{fs}:{fs+3}], %[rA] offset:{s * A_GROUP * 4 + buf * A_STAGE}",
            f"ds_read_b128 v[{fs+4}:{fs+7}], %[rB] offset:{s * 2048 + buf * B_STAGE}"]


def stage_stores(buf: int) -> list[str]:
    """v[80:91] into LDS buffer buf: each A float4 holds k = 4 q .. 4 q + 3 of
    one row and goes to four rows of group q (256 floats = 4 * 256 bytes
    apart, st64 units); the second A float4 is 128 rows (2 units) further;
    the B float4 is one 16-byte piece of a k-row."""
    u = buf * (A_STAGE // 256)
    return [f"ds_write2st64_b32 %[wA], v80, v81 offset0:{u + 0} offset1:{u + 4}",
            f"ds_write2st64_b32 %[wA], v82, v83 offset0:{u + 8} offset1:{u + 12}",
            f"ds_write2st64_b32 %[wA], v84, v85 offset0:{u + 2} offset1:{u + 6}",
            f"ds_write2st64_b32 %[wA], v86, v87 offset0:{u + 10} offset1:{u + 14}",
            f"ds_write_b128 %[wB], v[88:91] offset:{buf * B_STAGE}"]


LOADS = ["buffer_load_dwordx4 v[80:83], %[oA0], %[rsA], %[sA] offen",
         "buffer_load_dwordx4 v[84:87], %[oA1], %[rsA], %[sA] offen",
         "buffer_load_dwordx4 v[88:91], %[oB], %[rsB], %[sB] offen"]
ADVANCE = ["s_add_u32 %[sA], %[sA], 64", "s_add_u32 %[sB], %[sB], %[stepB]"]


def k_step(cur: int) -> list[str]:
    """One K step on LDS buffer cur; on entry set E is being read with step 0
    of this stage and v[80:91] are loading the next stage."""
    nxt = 1 - cur
    out = ["s_waitcnt lgkmcnt(0)", mfma(0, FE), *frag_reads(FO, 1, cur)]
    out += [mfma(b, FE) for b in (1, 2, 3)]
    out.append("s_waitcnt vmcnt(0)")
    stores = stage_stores(nxt)
    for b in range(4, 16):
        out.append(mfma(b, FE))
        if b < 4 + len(stores):
            out.append(stores[b - 4])
    # step 1 (set O); the stores above have completed once this wait is over,
    # so v[80:91] may take the stage after next
    out += ["s_waitcnt lgkmcnt(0)", mfma(0, FO), *frag_reads(FE, 2, cur)]
    for b in range(1, 16):
        out.append(mfma(b, FO))
        if b <= len(LOADS):
            out.append(LOADS[b - 1])
        if b == len(LOADS) + 1:
            out += ADVANCE
    # step 2 (set E)
    out += ["s_waitcnt lgkmcnt(0)", mfma(0, FE), *frag_reads(FO, 3, cur)]
    out += [mfma(b, FE) for b in range(1, 16)]
    # step 3 (set O): every wavefront's reads of this buffer and stores of
    # the next are complete at the barrier (lgkmcnt(0) before it)
    out += ["s_waitcnt lgkmcnt(0)"] + [mfma(b, FO) for b in range(8)]
    out += ["s_barrier", *frag_reads(FE, 0, nxt)]
    out += [mfma(b, FO) for b in range(8, 16)]
    return out


def program() -> list[str]:
    # stage 0 (the ragged remainder of K, or a whole stage) is stored into
    # buffer 0 by the kernel's C++ part just before this statement
    prologue = ["s_waitcnt lgkmcnt(0)", *LOADS, *ADVANCE, "s_barrier", *frag_reads(FE, 0, 0)]
    pairs = ["s_cmp_eq_u32 %[pairs], 0", "s_cbranch_scc1 .Lkloop_odd_%=", ".Lkloop_pair_%=:",
             *k_step(0), *k_step(1),
             "s_sub_u32 %[pairs], %[pairs], 1", "s_cmp_lg_u32 %[pairs], 0",
             "s_cbranch_scc1 .Lkloop_pair_%="]
    odd = [".Lkloop_odd_%=:", "s_cmp_eq_u32 %[odd], 0", "s_cbranch_scc1 .Lkloop_end_%=",
           *k_step(0), ".Lkloop_end_%=:"]
    # drain every load (v[64:91] are free after the asm statement) and give
    # the last MFMAs' results the wait states a vector read of them needs
    tail = ["s_waitcnt vmcnt(0) lgkmcnt(0)", "s_nop 7", "s_nop 7"]
    return prologue + pairs + odd + tail


def render() -> str:
    lines = ["// Generated by gen_kloop.py (the K loop of l10_kloop.hip); do not edit.",
             "#define SGEMM_KLOOP_ASM \\"]
    lines += [f'  "{ins}\\n" \\' for ins in program()]
    lines.append('  ""')
    return "\n".join(lines) + "\n"


if __name__ == "__main__":
    with open(OUT, "w") as f:
        f.write(render())
    print(OUT)
