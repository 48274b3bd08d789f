// l10_kloop.hip -- level 10's kernels for whole 256 x 128 and 128 x 128
// tiles: level 9's tile structure (64 x 64 wavefront tiles of 4 x 4
// 16 x 16 blocks, 16-deep K steps, double-buffered group-padded LDS,
// interleaved block rows and columns; eight or four wavefronts) with the K
// loop written as assembly (l10_kloop.inc, emitted by gen_kloop.py, which
// documents the schedule and the register map), for each orientation of
// the operands.
//
// [CP04] (section on boundary conditions and limits) attributes the last
// 15-20 % between a hand-written FP32 GEMM and the vendor library to
// instruction-level scheduling that compiled C++ does not reach; here that
// is the difference between level 9's compiled loop and this one on the
// same tile (4096^3: 138.5 against 150-152 TFLOP/s on MI355X).
//
// The first stage holds the K % 16 leftover k (a whole stage when
// K % 16 == 0), loaded with per-element bounds here in C++ and stored into
// LDS buffer 0 before the loop; every stage the loop loads is then whole.
// The loop reads A and B through buffer resources whose record counts end
// at the last element the tile may use, so the loads it issues past the
// last stage (one or two stages of prefetch) read zeros or elements of the
// same matrix, never beyond it; they land in the idle LDS buffer unused.
// Byte offsets must stay below 2^31 (kloop_fits).
//
// LDS holds both operands k-major whatever their storage (as level 9's
// tile): a row-major A and a transposed B arrive four k per 128-bit load
// and are transposed on their way in (into groups padded by 8 words), a
// transposed A and a row-major B arrive four m / n per load and are stored
// whole.  The fragments, the MFMAs and so the results are the same in every
// orientation.  With K % 16 == 0 they are bit-identical to level 9's
// 256 x 128 tile (the same blocks, the same operand values per MFMA, the
// same k order per accumulator); with a ragged K, level 9 takes the partial
// stage last and this kernel first.
#include "l10_kloop.inc"
#include "sgemm_internal.h"

namespace sgemm {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef int intx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

constexpr int round256(int n) { return (n + 255) / 256 * 256; }

// The tile constants gen_kloop.py builds each loop for.
template <int BM_, bool TA_, bool TB_>
struct KTile {
  static constexpr int BM = BM_, BN = 128, BK = 16, GROUP_M = 8;
  static constexpr bool TA = TA_, TB = TB_;
  static constexpr int WAVES_M = BM / 64, THREADS = 64 * 2 * WAVES_M;
  static constexpr int A_GROUP = 4 * BM + (TA ? 0 : 8);  // floats per four-k group
  static constexpr int B_GROUP = 4 * BN + (TB ? 8 : 0);
  static constexpr int A_STAGE = round256(4 * A_GROUP * 4);  // bytes per stage
  static constexpr int B_STAGE = round256(4 * B_GROUP * 4);
  static constexpr int LDS = 2 * A_STAGE + 2 * B_STAGE;
  static constexpr int A_LOADS = BM * BK / 4 / THREADS, B_LOADS = BK * BN / 4 / THREADS;
  static_assert(A_LOADS == 2 && (B_LOADS == 1 || B_LOADS == 2), "thread-to-element map");
  static_assert(THREADS / (BM / 4) == 8, "a transposed A's second float4 is 8 k-rows on");
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
  : [rsA] "s"(rsA), [rsB] "s"(rsB), [oA0] "v"(oA[0]), [oA1] "v"(oA[1]), [oB0] "v"(oB[0]),  \
    [oB1] "v"(oB[1]), [wA] "v"(wA), [wB] "v"(wB), [rA] "v"(rA), [rB] "v"(rB),              \
    [stepA] "s"(stepA), [stepB] "s"(stepB), [odd] "s"(odd)

#define SGEMM_KLOOP_RUN(NAME) \
  asm volatile(SGEMM_KLOOP_ASM_##NAME SGEMM_KLOOP_OPERANDS : SGEMM_KLOOP_CLOBBERS_##NAME, "memory", "scc")

// Per-thread element maps of one stage (the loop's loads and stores, and
// the C++ first stage, use the same ones).  Element h of a thread:
//   A row-major:  row tid/4 + h THREADS/4, k 4 (tid%4) .. +3
//   A transposed: k-row tid/(BM/4) + 8 h, rows 4 (tid%(BM/4)) .. +3
//   B row-major:  k-row tid/32 + h THREADS/32, columns 4 (tid%32) .. +3
//   B transposed: column tid/4 + h THREADS/4, k 4 (tid%4) .. +3
template <class T>
__device__ __forceinline__ void a_map(int tid, int h, int& row, int& k) {
  if (T::TA) {
    k = tid / (T::BM / 4) + 8 * h;
    row = 4 * (tid % (T::BM / 4));
  } else {
    row = tid / 4 + h * (T::THREADS / 4);
    k = 4 * (tid % 4);
  }
}
template <class T>
__device__ __forceinline__ void b_map(int tid, int h, int& k, int& col) {
  if (T::TB) {
    col = tid / 4 + h * (T::THREADS / 4);
    k = 4 * (tid % 4);
  } else {
    k = tid / 32 + h * (T::THREADS / 32);
    col = 4 * (tid % 32);
  }
}

// SPLIT (split K): work item i is K slice i / ntiles, k in
// [slice k_split, min(K, (slice + 1) k_split)), of tile i % ntiles, and
// stores its raw sums (no alpha, beta or C) into plane `slice` of ws, an
// M x N row-major array per slice; the reduction kernel adds the planes in
// slice order.
template <int BM, bool TA, bool TB, bool SPLIT>
__global__ __launch_bounds__((KTile<BM, TA, TB>::THREADS)) void k_kloop(Problem p, int64_t tiles_m,
                                                                       int64_t tiles_n,
                                                                       int64_t k_split,
                                                                       float* __restrict__ ws) {
  typedef KTile<BM, TA, TB> T;
  __shared__ __align__(16) char smem[T::LDS];
  const int64_t ntiles = tiles_m * tiles_n;
  const int64_t item = xcd_contiguous(blockIdx.x, gridDim.x);
  const int64_t t = SPLIT ? item % ntiles : item;
  const int64_t slice = SPLIT ? item / ntiles : 0;
  const int64_t k_lo = slice * k_split;
  const int K = SPLIT ? static_cast<int>(p.K - k_lo < k_split ? p.K - k_lo : k_split) : p.K;
  // tile order: XCD-contiguous ranges, grouped by GROUP_M rows of tiles
  const int64_t group = T::GROUP_M * tiles_n;
  const int64_t first_m = (t / group) * T::GROUP_M;
  const int64_t gm = tiles_m - first_m < T::GROUP_M ? tiles_m - first_m : T::GROUP_M;
  const int64_t in = t % group;
  const int64_t row0 = (first_m + in % gm) * BM;
  const int64_t col0 = (in / gm) * T::BN;

  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
  const int wm = wave / 2, wn = wave % 2, lrow = lane % 16, kg = lane / 16;
  const int64_t lda = p.lda, ldb = p.ldb;
  // The tile's part of A (rows row0 .. row0 + BM - 1, k_lo <= k < k_lo + K)
  // and of B (those k, columns col0 .. col0 + 127), as stored: element
  // (m, k_lo + k) of A at a_base[m a_rs + k a_ks], element (k_lo + k, n) of
  // B at b_base[k b_ks + n b_cs].
  const int64_t a_rs = TA ? 1 : lda, a_ks = TA ? lda : 1;
  const int64_t b_ks = TB ? 1 : ldb, b_cs = TB ? ldb : 1;
  const float* const a_base = p.A + row0 * a_rs + k_lo * a_ks;
  const float* const b_base = p.B + col0 * b_cs + k_lo * b_ks;
  const intx4 rsA =
      buffer_resource(a_base, static_cast<uint32_t>(((BM - 1) * a_rs + (K - 1) * a_ks + 1) * 4));
  const intx4 rsB =
      buffer_resource(b_base, static_cast<uint32_t>(((K - 1) * b_ks + (T::BN - 1) * b_cs + 1) * 4));
  uint32_t oA[2], oB[2] = {0, 0};
#pragma unroll
  for (int h = 0; h < T::A_LOADS; ++h) {
    int row, k;
    a_map<T>(tid, h, row, k);
    oA[h] = static_cast<uint32_t>((row * a_rs + k * a_ks) * 4);
  }
#pragma unroll
  for (int h = 0; h < T::B_LOADS; ++h) {
    int k, col;
    b_map<T>(tid, h, k, col);
    oB[h] = static_cast<uint32_t>((k * b_ks + col * b_cs) * 4);
  }
  // LDS: A stage k-row k at group k/4, word (k%4)*BM + m; B k-row k at
  // group k/4, word (k%4)*128 + n.  Stores start at element 0 of the
  // thread's map (element 1 is an immediate away); fragments of step s sit
  // in group s, a lane reading the four interleaved rows (columns)
  // 4 lrow .. 4 lrow + 3 of its wave tile at k-row kg of the step.
  const uint32_t base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_char*)smem));
  float* const lds_a = reinterpret_cast<float*>(smem);
  float* const lds_b = reinterpret_cast<float*>(smem + 2 * T::A_STAGE);
  int a_row0, a_k0, b_k0, b_col0;
  a_map<T>(tid, 0, a_row0, a_k0);
  b_map<T>(tid, 0, b_k0, b_col0);
  const int wa_word = (a_k0 / 4) * T::A_GROUP + (a_k0 % 4) * BM + a_row0;
  const int wb_word = (b_k0 / 4) * T::B_GROUP + (b_k0 % 4) * T::BN + b_col0;
  const uint32_t wA = base + static_cast<uint32_t>(wa_word * 4);
  const uint32_t wB = base + 2 * T::A_STAGE + static_cast<uint32_t>(wb_word * 4);
  const uint32_t rA = base + static_cast<uint32_t>((kg * BM + wm * 64 + 4 * lrow) * 4);
  const uint32_t rB =
      base + 2 * T::A_STAGE + static_cast<uint32_t>((kg * T::BN + wn * 64 + 4 * lrow) * 4);
  const uint32_t stepA = static_cast<uint32_t>(T::BK * a_ks * 4);
  const uint32_t stepB = static_cast<uint32_t>(T::BK * b_ks * 4);

  // stage 0: k < k0, into buffer 0 through the same element maps
  const int k0 = K % T::BK ? K % T::BK : T::BK;
  const float4 zero = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
  for (int h = 0; h < T::A_LOADS; ++h) {
    int row, k;
    a_map<T>(tid, h, row, k);
    if (TA) {
      // four rows of k-row k: whole or nothing
      const float4 v = k < k0 ? ld_global4(a_base + k * lda + row) : zero;
      *reinterpret_cast<float4*>(lds_a + (k / 4) * T::A_GROUP + (k % 4) * BM + row) = v;
    } else {
      // k .. k + 3 of one row, each below k0 or zero
      const float4 v = load4(a_base + row * lda, k, k0, true);
      float* const dst = lds_a + (k / 4) * T::A_GROUP + row;
      dst[0] = v.x;
      dst[BM] = v.y;
      dst[2 * BM] = v.z;
      dst[3 * BM] = v.w;
    }
  }
#pragma unroll
  for (int h = 0; h < T::B_LOADS; ++h) {
    int k, col;
    b_map<T>(tid, h, k, col);
    if (TB) {
      const float4 v = load4(b_base + col * ldb, k, k0, true);
      float* const dst = lds_b + (k / 4) * T::B_GROUP + col;
      dst[0] = v.x;
      dst[T::BN] = v.y;
      dst[2 * T::BN] = v.z;
      dst[3 * T::BN] = v.w;
    } else {
      const float4 v = k < k0 ? ld_global4(b_base + k * ldb + col) : zero;
      *reinterpret_cast<float4*>(lds_b + (k / 4) * T::B_GROUP + (k % 4) * T::BN + col) = v;
    }
  }
  uint32_t sA = static_cast<uint32_t>(k0 * a_ks * 4), sB = static_cast<uint32_t>(k0 * b_ks * 4);
  const int stages = (K + T::BK - 1) / T::BK;
  uint32_t pairs = static_cast<uint32_t>(stages / 2);
  const uint32_t odd = static_cast<uint32_t>(stages % 2);
  floatx16 a0 = {}, a1 = {}, a2 = {}, a3 = {};
  if constexpr (BM == 256 && !TA && !TB) SGEMM_KLOOP_RUN(256_NN);
  else if constexpr (BM == 256 && !TA) SGEMM_KLOOP_RUN(256_NT);
  else if constexpr (BM == 256 && !TB) SGEMM_KLOOP_RUN(256_TN);
  else if constexpr (BM == 256) SGEMM_KLOOP_RUN(256_TT);
  else if constexpr (!TA && !TB) SGEMM_KLOOP_RUN(128_NN);
  else if constexpr (!TA) SGEMM_KLOOP_RUN(128_NT);
  else if constexpr (!TB) SGEMM_KLOOP_RUN(128_TN);
  else SGEMM_KLOOP_RUN(128_TT);

  // Block (i, j) register r holds C[row0 + 64 wm + 16 kg + 4 r + i]
  // [col0 + 64 wn + 4 lrow + j]: for each (r, i) a lane owns four adjacent
  // outputs of one row.  With beta != 0 the four rows of one r are read
  // before any is written (the loads cannot move above earlier stores).
  const floatx16 acc[4] = {a0, a1, a2, a3};
  if (SPLIT) {
    float* const w = ws + slice * int64_t(p.M) * p.N + (row0 + wm * 64 + 16 * kg) * p.N + col0 +
                     wn * 64 + 4 * lrow;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        st_global4(w + (4 * r + i) * int64_t(p.N),
                   make_float4(acc[i][r], acc[i][4 + r], acc[i][8 + r], acc[i][12 + r]));
    return;
  }
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
  if (p.M <= 0 || p.N <= 0 || p.M % BM || p.N % 128 || p.K < 1) return false;
  // largest byte offset of a load (record counts, plus the stages the loop
  // prefetches past K: one for the 256-row tile, two for the 128-row one)
  // stays below 2^31
  const int64_t lim = int64_t(1) << 31, past = p.K + ((BM == 256 ? 1 : 2) + 1) * 16;
  const int64_t a_end = p.trans_a ? past * p.lda + BM : (BM - 1) * p.lda + past;
  const int64_t b_end = p.trans_b ? 127 * p.ldb + past : past * p.ldb + 128;
  return a_end * 4 < lim && b_end * 4 < lim;
}

template <int BM, bool TA, bool TB, bool SPLIT>
hipError_t launch_t(const Problem& p, int64_t k_split, float* ws, hipStream_t s) {
  typedef KTile<BM, TA, TB> T;
  const int64_t tm = p.M / BM, tn = p.N / T::BN;
  const int64_t items = tm * tn * (SPLIT ? ceil_div(p.K, k_split) : 1);
  hipLaunchKernelGGL((k_kloop<BM, TA, TB, SPLIT>), dim3(static_cast<unsigned>(items)),
                     dim3(T::THREADS), 0, s, p, tm, tn, k_split, ws);
  return hipGetLastError();
}

template <int BM, bool SPLIT>
hipError_t launch(const Problem& p, int64_t k_split, float* ws, hipStream_t s) {
  if (p.trans_a && p.trans_b) return launch_t<BM, true, true, SPLIT>(p, k_split, ws, s);
  if (p.trans_a) return launch_t<BM, true, false, SPLIT>(p, k_split, ws, s);
  if (p.trans_b) return launch_t<BM, false, true, SPLIT>(p, k_split, ws, s);
  return launch_t<BM, false, false, SPLIT>(p, k_split, ws, s);
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
  return shape == Shape::kHuge ? make_geometry(M, N, K, 256, 128, 16, 512)
                               : make_geometry(M, N, K, 128, 128, 16, 256);
}

hipError_t launch_tiles(Shape shape, const Problem& p, hipStream_t s) {
  if (!kloop_fits(shape, p)) return launch_mfma(shape, p, s);
  return shape == Shape::kHuge ? launch<256, false>(p, p.K, nullptr, s)
                               : launch<128, false>(p, p.K, nullptr, s);
}

Geometry tiles_split_geometry(Shape shape, int M, int N, int K, int64_t k_split) {
  Problem p{};
  p.M = M;
  p.N = N;
  p.K = K;
  p.lda = K;
  p.ldb = N;
  p.ldc = N;
  if (!kloop_fits(shape, p)) return mfma_split_geometry(shape, M, N, K, k_split);
  const int bm = shape == Shape::kHuge ? 256 : 128;
  Geometry g = make_geometry(M, N, K, bm, 128, 16, bm == 256 ? 512 : 256);
  g.tiles *= ceil_div(K, k_split);
  g.workgroups = g.tiles;
  g.k_steps = ceil_div(k_split, 16);
  return g;
}

hipError_t launch_tiles_split(Shape shape, const Problem& p, int64_t k_split, float* ws,
                              hipStream_t s) {
  if (!kloop_fits(shape, p)) return launch_mfma_split(shape, p, k_split, ws, s);
  return shape == Shape::kHuge ? launch<256, true>(p, k_split, ws, s)
                               : launch<128, true>(p, k_split, ws, s);
}

}  // namespace sgemm
