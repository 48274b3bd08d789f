// l10_kloop.hip -- level 10's kernel for whole 256 x 128 tiles: level 9's
// big tile (eight wavefronts of 4 x 4 16 x 16 blocks, 16-deep K steps,
// double-buffered group-padded LDS, interleaved block rows and columns)
// with its K loop written as assembly (l10_kloop.inc, emitted by
// gen_kloop.py, which documents the schedule and the register map).
//
// [CP04] (section on boundary conditions and limits) attributes the last
// 15-20 % between a hand-written FP32 GEMM and the vendor library to
// instruction-level scheduling that compiled C++ does not reach; here that
// is the difference between level 9's compiled loop and this one on the
// same tile (4096^3: 138.7 against 152 TFLOP/s on MI355X).
//
// The first stage holds the K % 16 leftover k (a whole stage when
// K % 16 == 0), loaded with per-element bounds here in C++ and stored into
// LDS buffer 0 before the loop; every stage the loop loads is then whole.
// The loop reads A and B through buffer resources whose record counts end
// at the last element the tile may use, so the loads it issues past the
// last stage (two stages of prefetch) read zeros or elements of the same
// matrix, never beyond it; they land in the idle LDS buffer unused.  The
// kernel takes row-major A and B and byte offsets below 2^31.
//
// With K % 16 == 0 the results are bit-identical to level 9's tile (the
// same blocks, the same operand values per MFMA, the same k order per
// accumulator); with a ragged K, level 9 takes the partial stage last and
// this kernel first, so the k order differs.
#include "l10_kloop.inc"
#include "sgemm_internal.h"

namespace sgemm {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef int intx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

constexpr int kBM = 256, kBN = 128, kBK = 16, kThreads = 512, kGroupM = 8;
constexpr int kAGroup = 4 * kBM + 8;              // floats per four-k group of A
constexpr int kAStage = 16640, kBStage = kBK * kBN * 4;  // bytes per LDS stage
constexpr int kLds = 2 * kAStage + 2 * kBStage;
static_assert(4 * kAGroup * 4 <= kAStage, "A stage holds four groups");

// Raw buffer resource (stride 0): loads at byte offsets >= bytes return 0.
__device__ __forceinline__ intx4 buffer_resource(const float* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  intx4 r;
  r.x = static_cast<int>(static_cast<uint32_t>(a));
  r.y = static_cast<int>(static_cast<uint32_t>(a >> 32) & 0xffffu);
  r.z = static_cast<int>(bytes);
  r.w = 0x00020000;  // 32-bit data format, as gfx9 raw buffer loads expect
  return r;
}

__global__ __launch_bounds__(kThreads) void k_kloop(Problem p, int64_t tiles_m, int64_t tiles_n) {
  __shared__ __align__(16) char smem[kLds];
  // tile order: XCD-contiguous ranges, grouped by GROUP_M rows of tiles
  const int64_t t = xcd_contiguous(blockIdx.x, gridDim.x);
  const int64_t group = kGroupM * tiles_n;
  const int64_t first_m = (t / group) * kGroupM;
  const int64_t gm = tiles_m - first_m < kGroupM ? tiles_m - first_m : kGroupM;
  const int64_t in = t % group;
  const int64_t row0 = (first_m + in % gm) * kBM;
  const int64_t col0 = (in / gm) * kBN;

  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
  const int wm = wave / 2, wn = wave % 2, lrow = lane % 16, kg = lane / 16;
  const int64_t lda = p.lda, ldb = p.ldb;
  // A: rows row0 .. row0 + 255, k < K; B: k < K, columns col0 .. col0 + 127
  const intx4 rsA = buffer_resource(p.A + row0 * lda, static_cast<uint32_t>(((kBM - 1) * lda + p.K) * 4));
  const intx4 rsB = buffer_resource(p.B + col0, static_cast<uint32_t>(((p.K - 1) * ldb + kBN) * 4));
  // loads of a stage: A float4s (row tid/4 and tid/4 + 128, k 4 (tid%4) ..),
  // B float4 (k-row tid/32, columns 4 (tid%32) ..)
  const uint32_t oA0 = static_cast<uint32_t>(((tid / 4) * lda + 4 * (tid % 4)) * 4);
  const uint32_t oA1 = oA0 + static_cast<uint32_t>(128 * lda * 4);
  const uint32_t oB = static_cast<uint32_t>(((tid / 32) * ldb + 4 * (tid % 32)) * 4);
  // LDS: A stage k-row k at group k/4, word (k%4)*256 + m; B k-row k at
  // word 128 k; fragments of step s at group s (A) / k-row 4 s (B), lane
  // reading the four interleaved rows (columns) 4 lrow .. 4 lrow + 3 of its
  // wave tile at k-row kg of the step
  const uint32_t base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_char*)smem));
  const uint32_t wA = base + static_cast<uint32_t>(((tid % 4) * kAGroup + tid / 4) * 4);
  const uint32_t wB = base + 2 * kAStage + static_cast<uint32_t>(tid * 16);
  const uint32_t rA = base + static_cast<uint32_t>((kg * kBM + wm * 64 + 4 * lrow) * 4);
  const uint32_t rB = base + 2 * kAStage + static_cast<uint32_t>((kg * kBN + wn * 64 + 4 * lrow) * 4);
  const uint32_t stepB = static_cast<uint32_t>(kBK * ldb * 4);
  // stage 0: k < k0 (the same thread-to-element map as the loop's stages)
  const int k0 = p.K % kBK ? p.K % kBK : kBK;
  {
    float* const lds = reinterpret_cast<float*>(smem);
    const float* const arow = p.A + (row0 + tid / 4) * lda;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float4 v = load4(arow + h * 128 * lda, 4 * (tid % 4), k0, true);
      float* const dst = lds + (tid % 4) * kAGroup + tid / 4 + 128 * h;
      dst[0] = v.x;
      dst[kBM] = v.y;
      dst[2 * kBM] = v.z;
      dst[3 * kBM] = v.w;
    }
    const int kb = tid / 32;
    const float4 bv = load4(p.B + (kb < k0 ? kb : 0) * ldb + col0, 4 * (tid % 32), kBN, kb < k0);
    *reinterpret_cast<float4*>(lds + 2 * kAStage / 4 + tid * 4) = bv;
  }
  uint32_t sA = static_cast<uint32_t>(k0 * 4), sB = static_cast<uint32_t>(k0 * ldb * 4);
  const int stages = (p.K + kBK - 1) / kBK;
  uint32_t pairs = static_cast<uint32_t>(stages / 2);
  const uint32_t odd = static_cast<uint32_t>(stages % 2);
  floatx16 a0 = {}, a1 = {}, a2 = {}, a3 = {};
  asm volatile(SGEMM_KLOOP_ASM
               : "+{v[0:15]}"(a0), "+{v[16:31]}"(a1), "+{v[32:47]}"(a2), "+{v[48:63]}"(a3),
                 [sA] "+s"(sA), [sB] "+s"(sB), [pairs] "+s"(pairs)
               : [rsA] "s"(rsA), [rsB] "s"(rsB), [oA0] "v"(oA0), [oA1] "v"(oA1), [oB] "v"(oB),
                 [wA] "v"(wA), [wB] "v"(wB), [rA] "v"(rA), [rB] "v"(rB), [stepB] "s"(stepB),
                 [odd] "s"(odd)
               : "v64", "v65", "v66", "v67", "v68", "v69", "v70", "v71", "v72", "v73", "v74",
                 "v75", "v76", "v77", "v78", "v79", "v80", "v81", "v82", "v83", "v84", "v85",
                 "v86", "v87", "v88", "v89", "v90", "v91", "memory", "scc");

  // Block (i, j) register r holds C[row0 + 64 wm + 16 kg + 4 r + i]
  // [col0 + 64 wn + 4 lrow + j]: for each (r, i) a lane owns four adjacent
  // outputs of one row.  With beta != 0 the four rows of one r are read
  // before any is written (the loads cannot move above earlier stores).
  const floatx16 acc[4] = {a0, a1, a2, a3};
  const float alpha = p.alpha, beta = p.beta;
  float* const cw = p.C + (row0 + wm * 64 + 16 * kg) * p.ldc + col0 + wn * 64 + 4 * lrow;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float4 old[4];
    if (beta != 0.0f) {
#pragma unroll
      for (int i = 0; i < 4; ++i) old[i] = ld_global4(cw + (4 * r + i) * p.ldc);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float4 v = make_float4(alpha * acc[i][r], alpha * acc[i][4 + r], alpha * acc[i][8 + r],
                             alpha * acc[i][12 + r]);
      if (beta != 0.0f) {
        v.x = fmaf(beta, old[i].x, v.x);
        v.y = fmaf(beta, old[i].y, v.y);
        v.z = fmaf(beta, old[i].z, v.z);
        v.w = fmaf(beta, old[i].w, v.w);
      }
      st_global4(cw + (4 * r + i) * p.ldc, v);
    }
  }
}

}  // namespace

bool kloop_fits(const Problem& p) {
  if (p.trans_a || p.trans_b || p.M <= 0 || p.N <= 0) return false;
  if (p.M % kBM || p.N % kBN || p.K < 1) return false;
  // largest byte offset of a load (record counts, plus the two stages the
  // loop prefetches past K) stays below 2^31
  const int64_t lim = int64_t(1) << 31;
  return ((kBM - 1) * p.lda + p.K + 2 * kBK) * 4 < lim &&
         ((p.K + 2 * kBK) * p.ldb + kBN) * 4 < lim;
}

hipError_t launch_kloop(const Problem& p, hipStream_t s) {
  if (!kloop_fits(p)) return hipErrorInvalidValue;
  const int64_t tm = p.M / kBM, tn = p.N / kBN;
  hipLaunchKernelGGL(k_kloop, dim3(static_cast<unsigned>(tm * tn)), dim3(kThreads), 0, s, p, tm, tn);
  return hipGetLastError();
}

hipError_t launch_tiles(Shape shape, const Problem& p, hipStream_t s) {
  if (shape == Shape::kHuge && kloop_fits(p)) return launch_kloop(p, s);
  return launch_mfma(shape, p, s);
}

}  // namespace sgemm
