// l10_kloop.hip -- level 10's kernels for whole 256 x 128 and 128 x 128
// tiles: level 9's tile structure (64 x 64 wavefront tiles of 4 x 4
// 16 x 16 blocks, 16-deep K steps, double-buffered group-padded LDS,
// interleaved block rows and columns; eight or four wavefronts) with the K
// loop written as assembly (l10_kloop.inc, emitted by gen_kloop.py, which
// documents the schedule and the register map).
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
// With K % 16 == 0 the 256 x 128 kernel's results are bit-identical to
// level 9's tile of that shape (the same blocks, the same operand values
// per MFMA, the same k order per accumulator); with a ragged K, level 9
// takes the partial stage last and this kernel first.
#include "l10_kloop.inc"
#include "sgemm_internal.h"

namespace sgemm {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef int intx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

// The tile constants gen_kloop.py builds each loop for.
template <int BM_>
struct KTile {
  static constexpr int BM = BM_, BN = 128, BK = 16, GROUP_M = 8;
  static constexpr int WAVES_M = BM / 64, THREADS = 64 * 2 * WAVES_M;
  static constexpr int A_GROUP = 4 * BM + 8;                          // floats per four-k group of A
  static constexpr int A_STAGE = (4 * A_GROUP * 4 + 255) / 256 * 256;  // bytes per A stage
  static constexpr int B_STAGE = BK * BN * 4;                          // bytes per B stage
  static constexpr int LDS = 2 * A_STAGE + 2 * B_STAGE;
  static constexpr int A_LOADS = BM * BK / 4 / THREADS, B_LOADS = BK * BN / 4 / THREADS;
  static constexpr int PREFETCH = BM == 256 ? 1 : 2;  // stages loaded ahead of the one stored
  static_assert(A_LOADS == 2 && (B_LOADS == 1 || B_LOADS == 2), "thread-to-element map");
};

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

#define SGEMM_KLOOP_OPERANDS                                                               \
  : "+{v[0:15]}"(a0), "+{v[16:31]}"(a1), "+{v[32:47]}"(a2), "+{v[48:63]}"(a3), [sA] "+s"(sA), \
    [sB] "+s"(sB), [pairs] "+s"(pairs)                                                     \
  : [rsA] "s"(rsA), [rsB] "s"(rsB), [oA0] "v"(oA0), [oA1] "v"(oA1), [oB0] "v"(oB0),        \
    [oB1] "v"(oB1), [wA] "v"(wA), [wB] "v"(wB), [rA] "v"(rA), [rB] "v"(rB),                \
    [stepB] "s"(stepB), [odd] "s"(odd)

template <int BM>
__global__ __launch_bounds__(KTile<BM>::THREADS) void k_kloop(Problem p, int64_t tiles_m,
                                                             int64_t tiles_n) {
  typedef KTile<BM> T;
  __shared__ __align__(16) char smem[T::LDS];
  // tile order: XCD-contiguous ranges, grouped by GROUP_M rows of tiles
  const int64_t t = xcd_contiguous(blockIdx.x, gridDim.x);
  const int64_t group = T::GROUP_M * tiles_n;
  const int64_t first_m = (t / group) * T::GROUP_M;
  const int64_t gm = tiles_m - first_m < T::GROUP_M ? tiles_m - first_m : T::GROUP_M;
  const int64_t in = t % group;
  const int64_t row0 = (first_m + in % gm) * BM;
  const int64_t col0 = (in / gm) * T::BN;

  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
  const int wm = wave / 2, wn = wave % 2, lrow = lane % 16, kg = lane / 16;
  const int64_t lda = p.lda, ldb = p.ldb;
  // A: rows row0 .. row0 + BM - 1, k < K; B: k < K, columns col0 .. col0 + 127
  const intx4 rsA = buffer_resource(p.A + row0 * lda, static_cast<uint32_t>(((BM - 1) * lda + p.K) * 4));
  const intx4 rsB = buffer_resource(p.B + col0, static_cast<uint32_t>(((p.K - 1) * ldb + T::BN) * 4));
  // loads of a stage: A float4 h at row tid/4 + h THREADS/4, k 4 (tid%4) ..;
  // B float4 h at k-row tid/32 + h THREADS/32, columns 4 (tid%32) ..
  constexpr int AROWS = T::THREADS / 4, BROWS = T::THREADS / 32;
  const uint32_t oA0 = static_cast<uint32_t>(((tid / 4) * lda + 4 * (tid % 4)) * 4);
  const uint32_t oA1 = oA0 + static_cast<uint32_t>(AROWS * lda * 4);
  const uint32_t oB0 = static_cast<uint32_t>(((tid / 32) * ldb + 4 * (tid % 32)) * 4);
  const uint32_t oB1 = oB0 + static_cast<uint32_t>(BROWS * ldb * 4);
  // LDS: A stage k-row k at group k/4, word (k%4)*BM + m; B k-row k at
  // word 128 k; fragments of step s at group s (A) / k-row 4 s (B), lane
  // reading the four interleaved rows (columns) 4 lrow .. 4 lrow + 3 of its
  // wave tile at k-row kg of the step
  const uint32_t base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_char*)smem));
  const uint32_t wA = base + static_cast<uint32_t>(((tid % 4) * T::A_GROUP + tid / 4) * 4);
  const uint32_t wB = base + 2 * T::A_STAGE + static_cast<uint32_t>(tid * 16);
  const uint32_t rA = base + static_cast<uint32_t>((kg * BM + wm * 64 + 4 * lrow) * 4);
  const uint32_t rB = base + 2 * T::A_STAGE + static_cast<uint32_t>((kg * T::BN + wn * 64 + 4 * lrow) * 4);
  const uint32_t stepB = static_cast<uint32_t>(T::BK * ldb * 4);
  // stage 0: k < k0 (the same thread-to-element map as the loop's stages)
  const int k0 = p.K % T::BK ? p.K % T::BK : T::BK;
  {
    float* const lds = reinterpret_cast<float*>(smem);
    const float* const arow = p.A + (row0 + tid / 4) * lda;
#pragma unroll
    for (int h = 0; h < T::A_LOADS; ++h) {
      const float4 v = load4(arow + h * AROWS * lda, 4 * (tid % 4), k0, true);
      float* const dst = lds + (tid % 4) * T::A_GROUP + tid / 4 + AROWS * h;
      dst[0] = v.x;
      dst[BM] = v.y;
      dst[2 * BM] = v.z;
      dst[3 * BM] = v.w;
    }
#pragma unroll
    for (int h = 0; h < T::B_LOADS; ++h) {
      const int kb = tid / 32 + BROWS * h;
      const float4 bv = load4(p.B + (kb < k0 ? kb : 0) * ldb + col0, 4 * (tid % 32), T::BN, kb < k0);
      *reinterpret_cast<float4*>(lds + 2 * T::A_STAGE / 4 + (tid + T::THREADS * h) * 4) = bv;
    }
  }
  uint32_t sA = static_cast<uint32_t>(k0 * 4), sB = static_cast<uint32_t>(k0 * ldb * 4);
  const int stages = (p.K + T::BK - 1) / T::BK;
  uint32_t pairs = static_cast<uint32_t>(stages / 2);
  const uint32_t odd = static_cast<uint32_t>(stages % 2);
  floatx16 a0 = {}, a1 = {}, a2 = {}, a3 = {};
  if constexpr (BM == 256) {
    asm volatile(SGEMM_KLOOP_ASM_256 SGEMM_KLOOP_OPERANDS
                 : SGEMM_KLOOP_CLOBBERS_256, "memory", "scc");
  } else {
    static_assert(BM == 128, "one loop per tile");
    asm volatile(SGEMM_KLOOP_ASM_128 SGEMM_KLOOP_OPERANDS
                 : SGEMM_KLOOP_CLOBBERS_128, "memory", "scc");
  }

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

template <int BM>
bool fits(const Problem& p) {
  typedef KTile<BM> T;
  if (p.trans_a || p.trans_b || p.M <= 0 || p.N <= 0) return false;
  if (p.M % BM || p.N % T::BN || p.K < 1) return false;
  // largest byte offset of a load (record counts, plus the stages the loop
  // prefetches past K) stays below 2^31
  const int64_t lim = int64_t(1) << 31, past = p.K + (T::PREFETCH + 1) * T::BK;
  return ((BM - 1) * p.lda + past) * 4 < lim && (past * p.ldb + T::BN) * 4 < lim;
}

template <int BM>
hipError_t launch(const Problem& p, hipStream_t s) {
  typedef KTile<BM> T;
  const int64_t tm = p.M / BM, tn = p.N / T::BN;
  hipLaunchKernelGGL(k_kloop<BM>, dim3(static_cast<unsigned>(tm * tn)), dim3(T::THREADS), 0, s, p,
                     tm, tn);
  return hipGetLastError();
}

}  // namespace

bool kloop_fits(Shape shape, const Problem& p) {
  switch (shape) {
    case Shape::kHuge: return fits<256>(p);
    case Shape::kLarge: return fits<128>(p);
    default: return false;
  }
}

Geometry tiles_geometry(Shape shape, int M, int N, int K) {
  Problem p{};
  p.M = M;
  p.N = N;
  p.K = K;
  p.lda = K;
  p.ldb = N;
  p.ldc = N;
  if (!kloop_fits(shape, p)) return mfma_geometry(shape, M, N, K);
  return shape == Shape::kHuge ? make_geometry(M, N, K, 256, 128, 16, KTile<256>::THREADS)
                               : make_geometry(M, N, K, 128, 128, 16, KTile<128>::THREADS);
}

hipError_t launch_tiles(Shape shape, const Problem& p, hipStream_t s) {
  if (!kloop_fits(shape, p)) return launch_mfma(shape, p, s);
  return shape == Shape::kHuge ? launch<256>(p, s) : launch<128>(p, s);
}

}  // namespace sgemm
