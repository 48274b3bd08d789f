// l10_kloop.hip -- level 10's kernels for whole 256 x 128, 128 x 128 and
// 64 x 64 tiles: level 9's tile structure (64 x 64 wavefront tiles of 4 x 4
// 16 x 16 blocks, double-buffered group-padded LDS, interleaved block rows
// and columns) with the K loop written as assembly (l10_kloop.inc, emitted
// by gen_kloop.py, which documents the schedule and the register map), for
// each orientation of the operands.  The 256 x 128 and 128 x 128 tiles take
// 16-deep stages, one wavefront per wave tile; the 64 x 64 tile takes
// 64-deep stages split over four wavefronts (each runs four of a stage's
// sixteen MFMA steps for the whole tile), whose sums meet in LDS after the
// loop, so that a tile with one wavefront per SIMD still has 64 MFMAs per
// wavefront between barriers.
//
// [CP04] (section on boundary conditions and limits) attributes the last
// 15-20 % between a hand-written FP32 GEMM and the vendor library to
// instruction-level scheduling that compiled C++ does not reach; here that
// is the difference between level 9's compiled loop and this one on the
// same tile (4096^3: 138.5 against 150-152 TFLOP/s on MI355X).
//
// The first stage holds the K % BK leftover k (a whole stage when
// K % BK == 0), loaded with per-element bounds here in C++ and stored into
// LDS buffer 0 before the loop; every stage the loop loads is then whole.
// The loop's first stages are requested by a prelude statement before the
// C++ loads of stage 0, so both memory latencies overlap.
// The loop reads A and B through buffer resources whose base is the next
// stage to load and whose record count ends at the last element the tile
// may use; each stage moves the base on and shrinks the count (down to 0),
// and the loads carry no scalar offset, so the hardware's range check on
// the per-thread offset bounds every load: the stages loaded past the last
// one (one or two of prefetch) read zeros without touching memory and land
// in the idle LDS buffer unused.  Byte offsets must stay below 2^31
// (kloop_fits).  Tiles at the bottom and
// right edges cover fewer rows / columns; their record counts stop at the
// last row / column of the matrix and their epilogue stores only inside it.
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
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef int intx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

constexpr int round256(int n) { return (n + 255) / 256 * 256; }

// The tile constants gen_kloop.py builds each loop for.
// GROUP_M: rows of tiles per group of the tile order, so that one XCD's
// contiguous run of tiles (its L2) covers GROUP_M tile rows.  The 256 x 128
// tile runs 64 tiles per XCD at once; 4 x 16 of them (A 1024 rows, B 2048
// columns) measured the fewest fabric fetches at 4096^3: 605 MB per call
// against 741 MB for 8 x 8 and 739 MB for 2 x 32, at the same time.
// FR: the fringe variant (one more row of C below the grid and / or one
// more column to its right, summed by the tiles' own blocks).
template <int BM_, int BN_, int BK_, int KS_, bool TA_, bool TB_, bool FR_ = false>
struct KTile {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, KS = KS_, GROUP_M = BM == 256 ? 4 : 8;
  static constexpr bool TA = TA_, TB = TB_, FR = FR_;
  static constexpr int WAVES_M = BM / 64, WAVES_N = BN / 64, WAVE_TILES = WAVES_M * WAVES_N;
  static constexpr int THREADS = 64 * WAVE_TILES * KS;
  static constexpr int GROUPS = BK / 4, STEPS = GROUPS / KS;  // MFMA steps per stage / per slice
  static constexpr int PAD = BK == 16 ? 8 : 4;  // words between four-k groups, transposing stores
  static constexpr int A_GROUP = 4 * BM + (TA ? 0 : PAD);  // floats per four-k group
  static constexpr int B_GROUP = 4 * BN + (TB ? PAD : 0);
  // bytes per stage; the fringe variant keeps BK + BK words after the
  // groups (the extra row's k, then the extra column's k)
  static constexpr int FPAD = GROUPS * A_GROUP * 4;
  static constexpr int A_STAGE = round256(FPAD + (FR ? 8 * BK : 0));
  // fringe variant: positions of a block's share per k (thread tid takes
  // k = tid / FP of each stage, position tid % FP)
  static constexpr int FP = THREADS / BK;
  static constexpr int B_STAGE = round256(GROUPS * B_GROUP * 4);
  static constexpr int STAGES_LDS = 2 * A_STAGE + 2 * B_STAGE;
  // K slices: each wavefront finishes 4 / KS block rows of its wave tile
  // and receives them from the other slices through LDS after the loop
  static constexpr int RED_FLOATS = KS > 1 ? WAVE_TILES * KS * KS * (4 / KS) * 16 * 64 : 0;
  static constexpr int LDS = STAGES_LDS > 4 * RED_FLOATS ? STAGES_LDS : 4 * RED_FLOATS;
  static constexpr int A_LOADS = BM * BK / 4 / THREADS, B_LOADS = BK * BN / 4 / THREADS;
  static constexpr int A_PER = TA ? BM / 4 : BK / 4;  // float4s per (k-)row of A as stored
  static constexpr int B_PER = TB ? BK / 4 : BN / 4;
  static constexpr int PREFETCH = BM * BN >= 256 * 128 ? 1 : 2;  // stages loaded ahead
  static_assert(A_LOADS >= 1 && A_LOADS <= 4 && B_LOADS >= 1 && B_LOADS <= 4, "loads per stage");
  static_assert(THREADS % A_PER == 0 && THREADS % B_PER == 0, "whole rows per load round");
  static_assert(4 % KS == 0 && STEPS >= 2, "K slices");
  static_assert(THREADS % BK == 0 && 3 * THREADS + BK <= STAGES_LDS / 4, "fringe shares and sums");
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

// The asm operands: the 16-deep tiles load two float4s of each operand per
// thread and stage (at most), the 64-deep tile four, and it also takes
// each buffer's own store base (its 32-bit stores cannot reach the second
// buffer by an immediate).  Unused inputs would still occupy registers.
// Two statements per tile: the prelude (stages 1 .. PREFETCH requested into
// the staging registers, its outputs) and the loop (the staging registers
// read-write, the accumulators pinned to v0 .. v63).  Both advance the
// buffer resources of A and B, pinned to s[60:63] and s[64:67] (the loop
// text names their words).
#define SGEMM_KLOOP_LOAD_INPUTS                                                  \
  [oA0] "v"(oA[0]), [oA1] "v"(oA[1]), [oB0] "v"(oB[0]), [stepA] "s"(stepA), \
      [stepB] "s"(stepB)
#define SGEMM_KLOOP_TWO_B , [oB1] "v"(oB[1])
#define SGEMM_KLOOP_ONE_B
#define SGEMM_KLOOP_DEEP \
  , [oB1] "v"(oB[1]), [oA2] "v"(oA[2]), [oA3] "v"(oA[3]), [oB2] "v"(oB[2]), [oB3] "v"(oB[3])
#define SGEMM_KLOOP_DEEP_STORES , [wA1] "v"(wA + T::A_STAGE), [wB1] "v"(wB + T::B_STAGE)
#define SGEMM_KLOOP_FRINGE_LOADS , [foa] "v"(foa), [fob] "v"(fob)
#define SGEMM_KLOOP_FRINGE_WORDS , [fst] "v"(fst), [frB] "v"(frB), [fcA] "v"(fcA), [fpk] "v"(fpk)
// the fringe variants' operands: the tile's own, then the fringe's
#define SGEMM_KLOOP_F2 SGEMM_KLOOP_TWO_B SGEMM_KLOOP_FRINGE_LOADS
#define SGEMM_KLOOP_F4 SGEMM_KLOOP_DEEP SGEMM_KLOOP_FRINGE_LOADS
#define SGEMM_KLOOP_FW SGEMM_KLOOP_FRINGE_WORDS
#define SGEMM_KLOOP_FW4 SGEMM_KLOOP_DEEP_STORES SGEMM_KLOOP_FRINGE_WORDS
#define SGEMM_KLOOP_PRELUDE(NAME, LOADS)                                                  \
  asm volatile(SGEMM_KLOOP_PRE_##NAME                                                     \
               : SGEMM_KLOOP_STAGING_OUT_##NAME, "+{s[60:63]}"(rsA), "+{s[64:67]}"(rsB)   \
               : SGEMM_KLOOP_LOAD_INPUTS LOADS                                            \
               : "memory", "scc")
#define SGEMM_KLOOP_LOOP(NAME, LOADS, STORES)                                             \
  asm volatile(SGEMM_KLOOP_ASM_##NAME                                                     \
               : "+{v[0:15]}"(a0), "+{v[16:31]}"(a1), "+{v[32:47]}"(a2), "+{v[48:63]}"(a3), \
                 "+{s[60:63]}"(rsA), "+{s[64:67]}"(rsB), [pairs] "+s"(pairs),             \
                 SGEMM_KLOOP_STAGING_IO_##NAME                                            \
               : SGEMM_KLOOP_LOAD_INPUTS LOADS STORES, [wA] "v"(wA), [wB] "v"(wB),       \
                 [rA] "v"(rA), [rB] "v"(rB), [odd] "s"(odd)                               \
               : SGEMM_KLOOP_CLOBBERS_##NAME, "memory", "scc")
// Per-thread element maps of one stage (the loop's loads and stores, and
// the C++ first stage, use the same ones).  Element h of a thread, with
// per = float4s per row (k-row) of the operand as stored (A_PER, B_PER) and
// (j, q) = stage_slot(tid):
//   A row-major:  row j + h THREADS/per, k 4 q .. 4 q + 3
//   A transposed: k-row j + h THREADS/per, rows 4 q .. 4 q + 3
//   B row-major:  k-row j + h THREADS/per, columns 4 q .. 4 q + 3
//   B transposed: column j + h THREADS/per, k 4 q .. 4 q + 3
// A 32-bit LDS store is served per half-wavefront, and words 32 apart share
// a bank there.  A transposing store (row-major A, transposed B) writes
// word 4 q + c of each of four k-rows of group q; with per == 16 (the
// 64-deep stage, groups 260 words apart, 4 mod 32) a half-wavefront takes
// 4 majors x 8 groups, whose 32 words fall in 32 banks (2 majors x 16
// groups would pair groups q and q + 8 on one bank).  Every other store
// takes consecutive groups of one major per lane run (tid / per, tid % per);
// either way a wavefront covers the same four majors, so its global loads
// read the same bytes.
template <int PER, bool TRANSPOSING>
__device__ __forceinline__ void stage_slot(int tid, int& j, int& q) {
  if constexpr (TRANSPOSING && PER == 16) {
    j = 4 * (tid / 64) + (tid / 8) % 4;
    q = tid % 8 + 8 * ((tid / 32) % 2);
  } else {
    j = tid / PER;
    q = tid % PER;
  }
}
template <class T>
__device__ __forceinline__ void a_map(int tid, int h, int& row, int& k) {
  int j, q;
  stage_slot<T::A_PER, !T::TA>(tid, j, q);
  const int major = j + h * (T::THREADS / T::A_PER), minor = 4 * q;
  row = T::TA ? minor : major;
  k = T::TA ? major : minor;
}
template <class T>
__device__ __forceinline__ void b_map(int tid, int h, int& k, int& col) {
  int j, q;
  stage_slot<T::B_PER, T::TB>(tid, j, q);
  const int major = j + h * (T::THREADS / T::B_PER), minor = 4 * q;
  k = T::TB ? minor : major;
  col = T::TB ? major : minor;
}

// SPLIT (split K): work item i is K part i / ntiles, k in
// [part k_split, min(K, (part + 1) k_split)), of tile i % ntiles, and
// stores its raw sums (no alpha, beta or C) into plane `part` of ws, an
// M x N row-major array per part; the reduction kernel adds the planes in
// part order.
// T::FR (the fringe variant): the tiles_m x tiles_n whole tiles cover all of
// C but row M - 1 when M = BM tiles_m + 1, and column N - 1 when
// N = BN tiles_n + 1.  Block (i, j) holds, over its K loop, op(A)'s rows
// of tile row i and op(B)'s columns of tile column j, all of K; so it also
// sums row M - 1 of op(A) against its share of those columns (columns
// i cpt .. i cpt + cpt - 1 of the tile, cpt = ceil(BN / tiles_m) <= FP)
// and its share of those rows (j rpt .., rpt = ceil(BM / tiles_n) <= FP)
// against column N - 1 of op(B), and the last block the corner: every
// output of the fringe is summed in one block, k = tid / FP of each stage
// per thread (the corner: k = tid % BK), and those BK partial sums are
// added in k order.  Row M - 1's and column N - 1's elements reach LDS
// with the stage they belong to; the block's record counts then reach
// that row / column.
template <class T, bool SPLIT>
__global__ __launch_bounds__(T::THREADS) void k_kloop(Problem p, int64_t tiles_m, int64_t tiles_n,
                                                      int64_t k_split, float* __restrict__ ws) {
  constexpr int BM = T::BM;
  constexpr bool TA = T::TA, TB = T::TB;
  __shared__ __align__(16) char smem[T::LDS];
  const int64_t ntiles = tiles_m * tiles_n;
  const int64_t item = xcd_contiguous(blockIdx.x, gridDim.x);
  const int64_t t = SPLIT ? item % ntiles : item;
  const int64_t part = SPLIT ? item / ntiles : 0;  // split-K part
  const int64_t k_lo = part * k_split;
  const int K = SPLIT ? static_cast<int>(p.K - k_lo < k_split ? p.K - k_lo : k_split) : p.K;
  // tile order: XCD-contiguous ranges, grouped by GROUP_M rows of tiles
  const int64_t group = T::GROUP_M * tiles_n;
  const int64_t first_m = (t / group) * T::GROUP_M;
  const int64_t gm = tiles_m - first_m < T::GROUP_M ? tiles_m - first_m : T::GROUP_M;
  const int64_t in = t % group;
  const int64_t row0 = (first_m + in % gm) * BM;
  const int64_t col0 = (in / gm) * T::BN;

  // rows / columns of C this tile covers (fewer than BM / BN at the edges)
  const int rows = static_cast<int>(p.M - row0 < BM ? p.M - row0 : BM);
  const int cols = static_cast<int>(p.N - col0 < T::BN ? p.N - col0 : T::BN);
  const bool whole = rows == BM && cols == T::BN;
  // fringe variant: the grid has row M - 1 / column N - 1 beside it (the
  // same for every block)
  const bool f_row = T::FR && p.M == tiles_m * BM + 1;
  const bool f_col = T::FR && p.N == tiles_n * T::BN + 1;

  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
  const int slice = wave / T::WAVE_TILES, wv = wave % T::WAVE_TILES;
  const int wm = wv / T::WAVES_N, wn = wv % T::WAVES_N, lrow = lane % 16, kg = lane / 16;
  const int64_t lda = p.lda, ldb = p.ldb;
  // The tile's part of A (rows row0 .. row0 + rows - 1, k_lo <= k < k_lo + K)
  // and of B (those k, columns col0 .. col0 + cols - 1), as stored: element
  // (m, k_lo + k) of A at a_base[m a_rs + k a_ks], element (k_lo + k, n) of
  // B at b_base[k b_ks + n b_cs].  The record counts end at the last of
  // these elements: at an edge tile the loads of rows (columns) beyond M
  // (N) read zeros, or elements of the same operand that only ever meet
  // outputs beyond M (N), which are not stored.
  const int64_t a_rs = TA ? 1 : lda, a_ks = TA ? lda : 1;
  const int64_t b_ks = TB ? 1 : ldb, b_cs = TB ? ldb : 1;
  const float* const a_base = p.A + row0 * a_rs + k_lo * a_ks;
  const float* const b_base = p.B + col0 * b_cs + k_lo * b_ks;
  // (fringe variant: rows / columns of the extra row / column, relative
  // to the tile, at which the record counts end where it exists)
  const int64_t a_last = f_row ? p.M - 1 - row0 : rows - 1;
  const int64_t b_last = f_col ? p.N - 1 - col0 : cols - 1;
  const uint32_t a_bytes = static_cast<uint32_t>((a_last * a_rs + (K - 1) * a_ks + 1) * 4);
  const uint32_t b_bytes = static_cast<uint32_t>(((K - 1) * b_ks + b_last * b_cs + 1) * 4);
  uint32_t oA[4] = {0, 0, 0, 0}, oB[4] = {0, 0, 0, 0};
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
  // group k/4, word (k%4)*BN + n.  Stores start at element 0 of the
  // thread's map (the others are immediates away); fragments of MFMA step
  // s sit in group s, a lane reading the four interleaved rows (columns)
  // 4 lrow .. 4 lrow + 3 of its wave tile at k-row kg of the step; a K
  // slice's steps start at group slice * STEPS.
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
  const int g0 = slice * T::STEPS;
  const uint32_t rA =
      base + static_cast<uint32_t>((g0 * T::A_GROUP + kg * BM + wm * 64 + 4 * lrow) * 4);
  const uint32_t rB = base + 2 * T::A_STAGE +
                      static_cast<uint32_t>((g0 * T::B_GROUP + kg * T::BN + wn * 64 + 4 * lrow) * 4);
  const uint32_t stepA = static_cast<uint32_t>(T::BK * a_ks * 4);
  const uint32_t stepB = static_cast<uint32_t>(T::BK * b_ks * 4);
  // fringe variant, per thread: the k of a stage it stages (tid % BK): the
  // byte offsets of element (a_last, k) of the tile's A and (k, b_last) of
  // its B; the k it multiplies (tid / FP) and the column n / row m of the
  // block's share it takes (tid % FP; beyond the share, a column / row of
  // the tile whose sums are not stored); its LDS bases: the staged words
  // of that k (extra row's at k, extra column's at BK + k), B's word (k, n),
  // A's word (m, k), and the staged words of k = tid % BK.
  const int64_t f_cpt = ceil_div(T::BN, tiles_m), f_rpt = ceil_div(BM, tiles_n);
  const int64_t f_n0 = (row0 / BM) * f_cpt, f_m0 = (col0 / T::BN) * f_rpt;
  uint32_t foa = 0, fob = 0, fst = 0, frB = 0, fcA = 0, fpk = 0;
  float fa[T::PREFETCH], fb[T::PREFETCH], frow = 0.0f, fcol = 0.0f, fcor = 0.0f;
  if constexpr (T::FR) {
    const int ks = tid % T::BK, kf = tid / T::FP, c = tid % T::FP;
    foa = static_cast<uint32_t>((a_last * a_rs + ks * a_ks) * 4);
    fob = static_cast<uint32_t>((ks * b_ks + b_last * b_cs) * 4);
    const int n = c < f_cpt && f_n0 + c < T::BN ? static_cast<int>(f_n0) + c : c;
    const int m = c < f_rpt && f_m0 + c < BM ? static_cast<int>(f_m0) + c : c;
    fst = base + static_cast<uint32_t>(4 * ks);
    fpk = base + static_cast<uint32_t>(4 * kf);
    frB = base + 2 * T::A_STAGE +
          static_cast<uint32_t>(((kf / 4) * T::B_GROUP + (kf % 4) * T::BN + n) * 4);
    fcA = base + static_cast<uint32_t>(((kf / 4) * T::A_GROUP + (kf % 4) * BM + m) * 4);
  }

  // stages 1 .. PREFETCH requested first (their loads stay in flight in the
  // staging registers), then stage 0: k < k0, into buffer 0 through the
  // same element maps (zeros beyond k0 and beyond the tile's rows /
  // columns); the two latencies overlap
  const int k0 = K % T::BK ? K % T::BK : T::BK;
  // the loop's resources start at stage 1 (k0 k on), their record counts
  // reduced by as much (0 when nothing of the tile is left)
  const int64_t a_skip = k0 * a_ks * 4, b_skip = k0 * b_ks * 4;
  intx4 rsA = buffer_resource(a_base + k0 * a_ks,
                              a_bytes > a_skip ? static_cast<uint32_t>(a_bytes - a_skip) : 0u);
  intx4 rsB = buffer_resource(b_base + k0 * b_ks,
                              b_bytes > b_skip ? static_cast<uint32_t>(b_bytes - b_skip) : 0u);
  floatx4 stg[T::PREFETCH * (T::A_LOADS + T::B_LOADS)];
  if constexpr (T::FR && BM == 256 && !TA && !TB) SGEMM_KLOOP_PRELUDE(256x128_NN_F, SGEMM_KLOOP_FRINGE_LOADS);
  else if constexpr (T::FR && BM == 256 && !TA) SGEMM_KLOOP_PRELUDE(256x128_NT_F, SGEMM_KLOOP_FRINGE_LOADS);
  else if constexpr (T::FR && BM == 256 && !TB) SGEMM_KLOOP_PRELUDE(256x128_TN_F, SGEMM_KLOOP_FRINGE_LOADS);
  else if constexpr (T::FR && BM == 256) SGEMM_KLOOP_PRELUDE(256x128_TT_F, SGEMM_KLOOP_FRINGE_LOADS);
  else if constexpr (T::FR && BM == 128 && !TA && !TB) SGEMM_KLOOP_PRELUDE(128x128_NN_F, SGEMM_KLOOP_F2);
  else if constexpr (T::FR && BM == 128 && !TA) SGEMM_KLOOP_PRELUDE(128x128_NT_F, SGEMM_KLOOP_F2);
  else if constexpr (T::FR && BM == 128 && !TB) SGEMM_KLOOP_PRELUDE(128x128_TN_F, SGEMM_KLOOP_F2);
  else if constexpr (T::FR && BM == 128) SGEMM_KLOOP_PRELUDE(128x128_TT_F, SGEMM_KLOOP_F2);
  else if constexpr (T::FR && !TA && !TB) SGEMM_KLOOP_PRELUDE(64x64_NN_F, SGEMM_KLOOP_F4);
  else if constexpr (T::FR && !TA) SGEMM_KLOOP_PRELUDE(64x64_NT_F, SGEMM_KLOOP_F4);
  else if constexpr (T::FR && !TB) SGEMM_KLOOP_PRELUDE(64x64_TN_F, SGEMM_KLOOP_F4);
  else if constexpr (T::FR) SGEMM_KLOOP_PRELUDE(64x64_TT_F, SGEMM_KLOOP_F4);
  else if constexpr (BM == 256 && !TA && !TB) SGEMM_KLOOP_PRELUDE(256x128_NN, SGEMM_KLOOP_ONE_B);
  else if constexpr (BM == 256 && !TA) SGEMM_KLOOP_PRELUDE(256x128_NT, SGEMM_KLOOP_ONE_B);
  else if constexpr (BM == 256 && !TB) SGEMM_KLOOP_PRELUDE(256x128_TN, SGEMM_KLOOP_ONE_B);
  else if constexpr (BM == 256) SGEMM_KLOOP_PRELUDE(256x128_TT, SGEMM_KLOOP_ONE_B);
  else if constexpr (BM == 128 && !TA && !TB) SGEMM_KLOOP_PRELUDE(128x128_NN, SGEMM_KLOOP_TWO_B);
  else if constexpr (BM == 128 && !TA) SGEMM_KLOOP_PRELUDE(128x128_NT, SGEMM_KLOOP_TWO_B);
  else if constexpr (BM == 128 && !TB) SGEMM_KLOOP_PRELUDE(128x128_TN, SGEMM_KLOOP_TWO_B);
  else if constexpr (BM == 128) SGEMM_KLOOP_PRELUDE(128x128_TT, SGEMM_KLOOP_TWO_B);
  else if constexpr (!TA && !TB) SGEMM_KLOOP_PRELUDE(64x64_NN, SGEMM_KLOOP_DEEP);
  else if constexpr (!TA) SGEMM_KLOOP_PRELUDE(64x64_NT, SGEMM_KLOOP_DEEP);
  else if constexpr (!TB) SGEMM_KLOOP_PRELUDE(64x64_TN, SGEMM_KLOOP_DEEP);
  else SGEMM_KLOOP_PRELUDE(64x64_TT, SGEMM_KLOOP_DEEP);
  // Stage 0 with buffer loads, all issued before the first LDS store (one
  // memory round trip, overlapping the prelude's); what lies outside the
  // stage (k >= k0) or the tile (rows, cols) is read at an offset beyond the
  // record count, which returns 0.  Whole tiles with k0 % 4 == 0 (a
  // uniform test) take each float4 whole or not at all (128-bit loads);
  // otherwise every element is its own 32-bit load.  The compiler sees
  // these loads and waits only as far as each store needs.
  constexpr uint32_t kOutside = 0x80000000u;  // beyond every record count (< 2^31)
  const __amdgpu_buffer_rsrc_t ra0 = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(a_base), 0, static_cast<int>(a_bytes), 0x00020000);
  const __amdgpu_buffer_rsrc_t rb0 = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(b_base), 0, static_cast<int>(b_bytes), 0x00020000);
  float av[T::A_LOADS][4], bv[T::B_LOADS][4];
  // fringe variant: stage 0's words of the extra row and column (zeros
  // beyond k0, and beyond the record counts where the block has none)
  float fa0 = 0.0f, fb0 = 0.0f;
  if constexpr (T::FR) {
    const bool in = tid % T::BK < k0;
    fa0 = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ra0, in ? foa : kOutside, 0, 0));
    fb0 = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rb0, in ? fob : kOutside, 0, 0));
  }
  if (k0 % 4 == 0 && whole) {
#pragma unroll
    for (int h = 0; h < T::A_LOADS; ++h) {
      int row, k;
      a_map<T>(tid, h, row, k);
      const uint32_t off = k < k0 ? static_cast<uint32_t>((row * a_rs + k * a_ks) * 4) : kOutside;
      const float4 v =
          __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(ra0, off, 0, 0));
      av[h][0] = v.x;
      av[h][1] = v.y;
      av[h][2] = v.z;
      av[h][3] = v.w;
    }
#pragma unroll
    for (int h = 0; h < T::B_LOADS; ++h) {
      int k, col;
      b_map<T>(tid, h, k, col);
      const uint32_t off = k < k0 ? static_cast<uint32_t>((k * b_ks + col * b_cs) * 4) : kOutside;
      const float4 v =
          __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rb0, off, 0, 0));
      bv[h][0] = v.x;
      bv[h][1] = v.y;
      bv[h][2] = v.z;
      bv[h][3] = v.w;
    }
  } else {
#pragma unroll
    for (int h = 0; h < T::A_LOADS; ++h) {
      int row, k;
      a_map<T>(tid, h, row, k);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        // a transposed A holds rows row .. row + 3 of k-row k, a row-major A
        // k .. k + 3 of row `row`
        const int r = TA ? row + c : row, kk = TA ? k : k + c;
        const uint32_t off =
            r < rows && kk < k0 ? static_cast<uint32_t>((r * a_rs + kk * a_ks) * 4) : kOutside;
        av[h][c] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ra0, off, 0, 0));
      }
    }
#pragma unroll
    for (int h = 0; h < T::B_LOADS; ++h) {
      int k, col;
      b_map<T>(tid, h, k, col);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        // a transposed B holds k .. k + 3 of column col, a row-major B
        // columns col .. col + 3 of k-row k
        const int kk = TB ? k + c : k, cc = TB ? col : col + c;
        const uint32_t off =
            cc < cols && kk < k0 ? static_cast<uint32_t>((kk * b_ks + cc * b_cs) * 4) : kOutside;
        bv[h][c] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rb0, off, 0, 0));
      }
    }
  }
#pragma unroll
  for (int h = 0; h < T::A_LOADS; ++h) {
    int row, k;
    a_map<T>(tid, h, row, k);
    if (TA) {
      *reinterpret_cast<float4*>(lds_a + (k / 4) * T::A_GROUP + (k % 4) * BM + row) =
          make_float4(av[h][0], av[h][1], av[h][2], av[h][3]);
    } else {
      float* const dst = lds_a + (k / 4) * T::A_GROUP + row;
#pragma unroll
      for (int c = 0; c < 4; ++c) dst[c * BM] = av[h][c];
    }
  }
#pragma unroll
  for (int h = 0; h < T::B_LOADS; ++h) {
    int k, col;
    b_map<T>(tid, h, k, col);
    if (TB) {
      float* const dst = lds_b + (k / 4) * T::B_GROUP + col;
#pragma unroll
      for (int c = 0; c < 4; ++c) dst[c * T::BN] = bv[h][c];
    } else {
      *reinterpret_cast<float4*>(lds_b + (k / 4) * T::B_GROUP + (k % 4) * T::BN + col) =
          make_float4(bv[h][0], bv[h][1], bv[h][2], bv[h][3]);
    }
  }
  if constexpr (T::FR) {
    // every thread of a k stores the same value
    float* const pad = lds_a + T::FPAD / 4;
    pad[tid % T::BK] = fa0;
    pad[T::BK + tid % T::BK] = fb0;
  }
  const int stages = (K + T::BK - 1) / T::BK;
  uint32_t pairs = static_cast<uint32_t>(stages / 2);
  const uint32_t odd = static_cast<uint32_t>(stages % 2);
  floatx16 a0 = {}, a1 = {}, a2 = {}, a3 = {};
  if constexpr (T::FR && BM == 256 && !TA && !TB) SGEMM_KLOOP_LOOP(256x128_NN_F, SGEMM_KLOOP_FRINGE_LOADS, SGEMM_KLOOP_FW);
  else if constexpr (T::FR && BM == 256 && !TA) SGEMM_KLOOP_LOOP(256x128_NT_F, SGEMM_KLOOP_FRINGE_LOADS, SGEMM_KLOOP_FW);
  else if constexpr (T::FR && BM == 256 && !TB) SGEMM_KLOOP_LOOP(256x128_TN_F, SGEMM_KLOOP_FRINGE_LOADS, SGEMM_KLOOP_FW);
  else if constexpr (T::FR && BM == 256) SGEMM_KLOOP_LOOP(256x128_TT_F, SGEMM_KLOOP_FRINGE_LOADS, SGEMM_KLOOP_FW);
  else if constexpr (T::FR && BM == 128 && !TA && !TB) SGEMM_KLOOP_LOOP(128x128_NN_F, SGEMM_KLOOP_F2, SGEMM_KLOOP_FW);
  else if constexpr (T::FR && BM == 128 && !TA) SGEMM_KLOOP_LOOP(128x128_NT_F, SGEMM_KLOOP_F2, SGEMM_KLOOP_FW);
  else if constexpr (T::FR && BM == 128 && !TB) SGEMM_KLOOP_LOOP(128x128_TN_F, SGEMM_KLOOP_F2, SGEMM_KLOOP_FW);
  else if constexpr (T::FR && BM == 128) SGEMM_KLOOP_LOOP(128x128_TT_F, SGEMM_KLOOP_F2, SGEMM_KLOOP_FW);
  else if constexpr (T::FR && !TA && !TB) SGEMM_KLOOP_LOOP(64x64_NN_F, SGEMM_KLOOP_F4, SGEMM_KLOOP_FW4);
  else if constexpr (T::FR && !TA) SGEMM_KLOOP_LOOP(64x64_NT_F, SGEMM_KLOOP_F4, SGEMM_KLOOP_FW4);
  else if constexpr (T::FR && !TB) SGEMM_KLOOP_LOOP(64x64_TN_F, SGEMM_KLOOP_F4, SGEMM_KLOOP_FW4);
  else if constexpr (T::FR) SGEMM_KLOOP_LOOP(64x64_TT_F, SGEMM_KLOOP_F4, SGEMM_KLOOP_FW4);
  else if constexpr (BM == 256 && !TA && !TB) SGEMM_KLOOP_LOOP(256x128_NN, SGEMM_KLOOP_ONE_B, );
  else if constexpr (BM == 256 && !TA) SGEMM_KLOOP_LOOP(256x128_NT, SGEMM_KLOOP_ONE_B, );
  else if constexpr (BM == 256 && !TB) SGEMM_KLOOP_LOOP(256x128_TN, SGEMM_KLOOP_ONE_B, );
  else if constexpr (BM == 256) SGEMM_KLOOP_LOOP(256x128_TT, SGEMM_KLOOP_ONE_B, );
  else if constexpr (BM == 128 && !TA && !TB) SGEMM_KLOOP_LOOP(128x128_NN, SGEMM_KLOOP_TWO_B, );
  else if constexpr (BM == 128 && !TA) SGEMM_KLOOP_LOOP(128x128_NT, SGEMM_KLOOP_TWO_B, );
  else if constexpr (BM == 128 && !TB) SGEMM_KLOOP_LOOP(128x128_TN, SGEMM_KLOOP_TWO_B, );
  else if constexpr (BM == 128) SGEMM_KLOOP_LOOP(128x128_TT, SGEMM_KLOOP_TWO_B, );
  else if constexpr (!TA && !TB) SGEMM_KLOOP_LOOP(64x64_NN, SGEMM_KLOOP_DEEP, SGEMM_KLOOP_DEEP_STORES);
  else if constexpr (!TA) SGEMM_KLOOP_LOOP(64x64_NT, SGEMM_KLOOP_DEEP, SGEMM_KLOOP_DEEP_STORES);
  else if constexpr (!TB) SGEMM_KLOOP_LOOP(64x64_TN, SGEMM_KLOOP_DEEP, SGEMM_KLOOP_DEEP_STORES);
  else SGEMM_KLOOP_LOOP(64x64_TT, SGEMM_KLOOP_DEEP, SGEMM_KLOOP_DEEP_STORES);
  floatx16 acc[4] = {a0, a1, a2, a3};

  // fringe variant: the partial sums meet in LDS (free once every
  // wavefront has left the loop), one per k of a stage for each output.
  // Each output adds its BK in a fixed order: in groups of G consecutive k
  // (G = BK up to 16, else 8), then the groups in order -- the block's
  // share of row M - 1 at share positions 0 .. FP - 1, of column N - 1 at
  // FP .. 2 FP - 1, and in the last block the corner at 2 FP.
  if constexpr (T::FR) {
    if (f_row || f_col) {
      constexpr int FP = T::FP, G = T::BK <= 16 ? T::BK : 8, NG = T::BK / G;
      static_assert(T::BK % G == 0 && (2 * FP + 1) * NG <= T::THREADS, "fringe sums");
      float* const red = reinterpret_cast<float*>(smem);
      float* const part = red + 2 * T::THREADS + T::BK;  // NG group sums per output
      __syncthreads();
      red[tid] = frow;
      red[T::THREADS + tid] = fcol;
      if (tid < T::BK) red[2 * T::THREADS + tid] = fcor;
      __syncthreads();
      // thread (o, g): output o (row share positions, column share
      // positions, corner), group g of its k
      const int o = tid / NG, g = tid % NG;
      if (o <= 2 * FP) {
        const float* const src = o < FP ? red + o : o < 2 * FP ? red + T::THREADS + (o - FP) : red + 2 * T::THREADS;
        const int stride = o < 2 * FP ? FP : 1;
        float sum = src[stride * (g * G)];
        for (int k = 1; k < G; ++k) sum += src[stride * (g * G + k)];
        part[o * NG + g] = sum;
      }
      if constexpr (NG > 1) __syncthreads();
      auto total = [&](int out) {
        float sum = part[out * NG];
        for (int q = 1; q < NG; ++q) sum += part[out * NG + q];
        return sum;
      };
      if (f_row && tid < FP && tid < f_cpt && f_n0 + tid < T::BN) {
        float* const c = p.C + int64_t(p.M - 1) * p.ldc + col0 + f_n0 + tid;
        *c = epilogue(total(tid), p.alpha, p.beta, c);
      }
      const int r = tid - FP;
      if (f_col && r >= 0 && r < FP && r < f_rpt && f_m0 + r < BM) {
        float* const c = p.C + (row0 + f_m0 + r) * p.ldc + (p.N - 1);
        *c = epilogue(total(tid), p.alpha, p.beta, c);
      }
      if (f_row && f_col && tid == 2 * FP && t == tiles_m * tiles_n - 1) {
        float* const c = p.C + int64_t(p.M - 1) * p.ldc + (p.N - 1);
        *c = epilogue(total(tid), p.alpha, p.beta, c);
      }
    }
  }

  // K slices: slice s finishes block rows i with i / (4 / KS) == s.  Every
  // wavefront writes the block rows the others finish into LDS (lane-
  // contiguous, conflict free; the stage buffers are free once every
  // wavefront has left the loop), then adds what it receives in slice
  // order: ((p_0 + p_1) + p_2) + p_3, the same order for every output.
  int ilo = 0, ihi = 4;
  if constexpr (T::KS > 1) {
    constexpr int RPS = 4 / T::KS;  // block rows per slice
    float* const red = reinterpret_cast<float*>(smem);
    // red[wave tile][destination slice][source slice][row][register][lane]
    auto at = [&](int dst, int src, int row, int e) {
      return (((((wv * T::KS + dst) * T::KS + src) * RPS + row) * 16 + e) * 64) + lane;
    };
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int dst = i / RPS;
      if (dst == slice) continue;
#pragma unroll
      for (int e = 0; e < 16; ++e) red[at(dst, slice, i % RPS, e)] = acc[i][e];
    }
    __syncthreads();
    ilo = slice * RPS;
    ihi = ilo + RPS;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i < ilo || i >= ihi) continue;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float sum = slice == 0 ? acc[i][e] : red[at(slice, 0, i % RPS, e)];
#pragma unroll
        for (int src = 1; src < T::KS; ++src) sum += src == slice ? acc[i][e] : red[at(slice, src, i % RPS, e)];
        acc[i][e] = sum;
      }
    }
  }

  // Block (i, j) register r holds C[row0 + 64 wm + 16 kg + 4 r + i]
  // [col0 + 64 wn + 4 lrow + j]: for each (r, i) a lane owns four adjacent
  // outputs of one row.  With beta != 0 the rows of one r are read before
  // any is written (the loads cannot move above earlier stores).  Edge
  // tiles store only rows below M and columns below N.
  const int r_lane = wm * 64 + 16 * kg, c_lane = wn * 64 + 4 * lrow;  // within the tile
  if (SPLIT) {
    float* const w = ws + part * int64_t(p.M) * p.N + (row0 + r_lane) * p.N + col0 + c_lane;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i < ilo || i >= ihi || r_lane + 4 * r + i >= rows) continue;
        const float4 v = make_float4(acc[i][r], acc[i][4 + r], acc[i][8 + r], acc[i][12 + r]);
        float* const wr = w + (4 * r + i) * int64_t(p.N);
        if (whole || c_lane + 3 < cols) {
          st_global4(wr, v);
        } else {
          if (c_lane + 0 < cols) wr[0] = v.x;
          if (c_lane + 1 < cols) wr[1] = v.y;
          if (c_lane + 2 < cols) wr[2] = v.z;
        }
      }
    return;
  }
  const float alpha = p.alpha, beta = p.beta;
  float* const cw = p.C + (row0 + r_lane) * p.ldc + col0 + c_lane;
  if (!whole) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (i >= ilo && i < ihi && r_lane + 4 * r + i < rows)
          store4(cw + (4 * r + i) * p.ldc, c_lane, cols,
                 make_float4(acc[i][r], acc[i][4 + r], acc[i][8 + r], acc[i][12 + r]), alpha, beta);
    return;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float4 old[4];
    if (beta != 0.0f) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (i >= ilo && i < ihi) old[i] = ld_global4(cw + (4 * r + i) * p.ldc);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i < ilo || i >= ihi) continue;
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

template <class T>
bool fits(const Problem& p) {
  if (p.trans_a != T::TA || p.trans_b != T::TB) return false;
  if (p.M <= 0 || p.N <= 0 || p.K < 1) return false;
  // largest byte offset of a load (record counts, plus the stages the loop
  // prefetches past K) stays below 2^31
  const int64_t lim = int64_t(1) << 31, past = p.K + (T::PREFETCH + 1) * T::BK;
  const int64_t a_end = T::TA ? past * p.lda + T::BM : (T::BM - 1) * p.lda + past;
  const int64_t b_end = T::TB ? (T::BN - 1) * p.ldb + past : past * p.ldb + T::BN;
  return a_end * 4 < lim && b_end * 4 < lim;
}

// The fringe variant over a grid of Mm x Nm (whole tiles) inside p, with
// p.M - Mm and p.N - Nm each 0 or 1: enough tile rows and columns that
// each block's share of the fringe is at most FP columns / rows (256 x 128:
// 4 x 8 tiles, 128 x 128: 8 x 8, 64 x 64: 16 x 16), and every block's
// offsets down to row M - 1 / across to column N - 1 (largest from the
// first tile) below 2^31 bytes.
template <class T>
bool fits_fringe(const Problem& p, int Mm, int Nm) {
  if (p.trans_a != T::TA || p.trans_b != T::TB) return false;
  if (Mm < T::BM || Nm < T::BN || Mm % T::BM || Nm % T::BN || p.K < 1) return false;
  if (ceil_div(T::BN, Mm / T::BM) > T::FP || ceil_div(T::BM, Nm / T::BN) > T::FP) return false;
  if (p.M - Mm < 0 || p.M - Mm > 1 || p.N - Nm < 0 || p.N - Nm > 1) return false;
  const int64_t lim = int64_t(1) << 31, past = p.K + (T::PREFETCH + 1) * T::BK;
  const int64_t a_end = T::TA ? past * p.lda + p.M : (p.M - 1) * p.lda + past;
  const int64_t b_end = T::TB ? (p.N - 1) * p.ldb + past : past * p.ldb + p.N;
  return a_end * 4 < lim && b_end * 4 < lim;
}

template <class T, bool SPLIT>
hipError_t launch_t(const Problem& p, int64_t k_split, float* ws, hipStream_t s) {
  const int64_t tm = ceil_div(p.M, T::BM), tn = ceil_div(p.N, T::BN);
  const int64_t items = tm * tn * (SPLIT ? ceil_div(p.K, k_split) : 1);
  hipLaunchKernelGGL((k_kloop<T, SPLIT>), dim3(static_cast<unsigned>(items)), dim3(T::THREADS), 0, s,
                     p, tm, tn, k_split, ws);
  return hipGetLastError();
}

// The tile of each shape (orientation as given); f(tile type) is called
// with the one that applies.
template <int BM, int BN, int BK, int KS, class F>
auto with_orientation(const Problem& p, F f) {
  if (p.trans_a && p.trans_b) return f(KTile<BM, BN, BK, KS, true, true>());
  if (p.trans_a) return f(KTile<BM, BN, BK, KS, true, false>());
  if (p.trans_b) return f(KTile<BM, BN, BK, KS, false, true>());
  return f(KTile<BM, BN, BK, KS, false, false>());
}

template <int BM, int BN, int BK, int KS, class F>
auto with_fringe_orientation(const Problem& p, F f) {
  if (p.trans_a && p.trans_b) return f(KTile<BM, BN, BK, KS, true, true, true>());
  if (p.trans_a) return f(KTile<BM, BN, BK, KS, true, false, true>());
  if (p.trans_b) return f(KTile<BM, BN, BK, KS, false, true, true>());
  return f(KTile<BM, BN, BK, KS, false, false, true>());
}

// The fringe variant of each loop tile (has_loop(shape) must hold).
template <class F>
auto with_fringe_tile(Shape shape, const Problem& p, F f) {
  switch (shape) {
    case Shape::kHuge: return with_fringe_orientation<256, 128, 16, 1>(p, f);
    case Shape::kLarge: return with_fringe_orientation<128, 128, 16, 1>(p, f);
    default: return with_fringe_orientation<64, 64, 64, 4>(p, f);
  }
}

template <class F>
auto with_tile(Shape shape, const Problem& p, F f) {
  switch (shape) {
    case Shape::kHuge: return with_orientation<256, 128, 16, 1>(p, f);
    case Shape::kLarge: return with_orientation<128, 128, 16, 1>(p, f);
    default: return with_orientation<64, 64, 64, 4>(p, f);
  }
}

bool has_loop(Shape shape) {
  return shape == Shape::kHuge || shape == Shape::kLarge || shape == Shape::kSmallDeep;
}

// The compiled tile that stands in where a loop kernel does not fit.
Shape compiled(Shape shape) { return shape == Shape::kSmallDeep ? Shape::kSmallSliced : shape; }

}  // namespace

bool kloop_fits(Shape shape, const Problem& p) {
  return has_loop(shape) && with_tile(shape, p, [&](auto t) { return fits<decltype(t)>(p); });
}

Geometry tiles_geometry(Shape shape, int M, int N, int K) {
  Problem p{};
  p.M = M;
  p.N = N;
  p.K = K;
  p.lda = K;
  p.ldb = N;
  p.ldc = N;
  if (!kloop_fits(shape, p)) return mfma_geometry(compiled(shape), M, N, K);
  return with_tile(shape, p, [&](auto t) {
    typedef decltype(t) T;
    return make_geometry(M, N, K, T::BM, T::BN, T::BK, T::THREADS);
  });
}

hipError_t launch_tiles(Shape shape, const Problem& p, hipStream_t s) {
  if (!kloop_fits(shape, p)) return launch_mfma(compiled(shape), p, s);
  return with_tile(shape, p, [&](auto t) { return launch_t<decltype(t), false>(p, p.K, nullptr, s); });
}

bool tiles_fringe_fits(Shape shape, const Problem& p, int Mm, int Nm) {
  return has_loop(shape) &&
         with_fringe_tile(shape, p, [&](auto t) { return fits_fringe<decltype(t)>(p, Mm, Nm); });
}

hipError_t launch_tiles_fringe(Shape shape, const Problem& p, int Mm, int Nm, hipStream_t s) {
  if (!tiles_fringe_fits(shape, p, Mm, Nm)) return hipErrorInvalidValue;
  return with_fringe_tile(shape, p, [&](auto t) {
    typedef decltype(t) T;
    const int64_t tm = Mm / T::BM, tn = Nm / T::BN;
    hipLaunchKernelGGL((k_kloop<T, false>), dim3(static_cast<unsigned>(tm * tn)), dim3(T::THREADS), 0, s,
                       p, tm, tn, int64_t(p.K), nullptr);
    return hipGetLastError();
  });
}

Geometry tiles_split_geometry(Shape shape, int M, int N, int K, int64_t k_split) {
  Problem p{};
  p.M = M;
  p.N = N;
  p.K = K;
  p.lda = K;
  p.ldb = N;
  p.ldc = N;
  if (!kloop_fits(shape, p)) return mfma_split_geometry(compiled(shape), M, N, K, k_split);
  return with_tile(shape, p, [&](auto t) {
    typedef decltype(t) T;
    Geometry g = make_geometry(M, N, K, T::BM, T::BN, T::BK, T::THREADS);
    g.tiles *= ceil_div(K, k_split);
    g.workgroups = g.tiles;
    g.k_steps = ceil_div(k_split, T::BK);
    return g;
  });
}

hipError_t launch_tiles_split(Shape shape, const Problem& p, int64_t k_split, float* ws,
                              hipStream_t s) {
  if (!kloop_fits(shape, p)) return launch_mfma_split(compiled(shape), p, k_split, ws, s);
  return with_tile(shape, p, [&](auto t) { return launch_t<decltype(t), true>(p, k_split, ws, s); });
}

}  // namespace sgemm
