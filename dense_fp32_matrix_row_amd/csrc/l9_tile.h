// l9_tile.h -- the matrix-core tile kernel of levels 9 and 10 (internal
// header: the kernel template, its launchers and the tile shapes; each
// source that includes it instantiates the operand orientations it needs).
//
// Block tile BM x BN with BK-deep K steps and WAVES_M x WAVES_N wavefronts
// (times KSLICE K slices), each owning a WTM x WTN wave tile made of
// BLK_M x BLK_N MFMA blocks, 32 x 32 (v_mfma_f32_32x32x2_f32, 2048 FMAs) or
// 16 x 16 (v_mfma_f32_16x16x4_f32, 1024 FMAs); full float32 inputs and
// accumulators either way.
//
// Operand layout (MfmaOp below): lane l supplies A[l % DIM][l / DIM] and
// B[l / DIM][l % DIM]; for 32 x 32 accumulator register r of lane l holds
// C[8*(r/4) + 4*(l/32) + r%4][l % 32], for 16 x 16 C[4*(l/16) + r][l % 16].
// Rows and columns of the wave tile
// are interleaved over the blocks: MFMA row i of block bi is wave-tile row
// BLK_M*i + bi (columns likewise), so the BLK_M A values a lane needs for one
// k are adjacent in the k-major LDS tile (one 64-bit read for BLK_M = 2),
// and a lane's BLK_N outputs of one row are adjacent in C (one 64-bit store).
// MFMA step s of a K-phase consumes k = KPER*s + l/DIM (KPER = 2 or 4).
//
// LDS holds both operands k-major, k-row k of A at As[k / 4][(k % 4) * BM + m]
// (likewise B): unpadded rows in groups of four, the groups a few words
// apart (Panel below gives the bank arithmetic).  A row-major A (and a
// transposed B, stored N x K) arrive 4 consecutive k per 128-bit load and
// are transposed on their way into LDS; a transposed A (stored K x M) and a
// row-major B arrive 4 consecutive m / n per load and are copied as is.
#pragma once

#include <type_traits>

#include "sgemm_internal.h"

namespace sgemm {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// The two FP32 matrix instructions, one 32 x 32 or 16 x 16 block each (the
// same 64 FLOP per SIMD per cycle): lane l supplies A[l % DIM][l / DIM] and
// B[l / DIM][l % DIM] (KPER = 64 / DIM k values per instruction), and its
// accumulator register r holds C[row(l / DIM, r)][l % DIM].
template <int MS>
struct MfmaOp;
template <>
struct MfmaOp<32> {  // v_mfma_f32_32x32x2_f32: 16 passes
  static constexpr int DIM = 32, KPER = 2, REGS = 16;
  typedef floatx16 acc_t;
  __device__ static acc_t mma(float a, float b, const acc_t& c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  __host__ __device__ static constexpr int row(int g, int r) { return 8 * (r / 4) + 4 * g + r % 4; }
};
template <>
struct MfmaOp<16> {  // v_mfma_f32_16x16x4_f32: 8 passes
  static constexpr int DIM = 16, KPER = 4, REGS = 4;
  typedef floatx4 acc_t;
  __device__ static acc_t mma(float a, float b, const acc_t& c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  __host__ __device__ static constexpr int row(int g, int r) { return 4 * g + r; }
};


// A tile configuration: BM x BN block tile, BK-deep K steps, WAVES_M x
// WAVES_N wavefronts (each owning a (BM/WAVES_M) x (BN/WAVES_N) wave tile),
// how many of a K step's BK/2 MFMA steps are unrolled together (fewer keeps
// the compiler from hoisting every fragment read into registers), how many
// tile-rows one group of the block order spans, whether wavefronts raise
// their issue priority around the barrier (PRIO, below), and into how many
// K slices each stage is cut (KSLICE: KSLICE x WAVES_M x WAVES_N wavefronts;
// slice j takes MFMA steps [j, j+1) * BK/2/KSLICE of every stage, and the
// slices' sums meet in LDS after the K loop, added in slice order).  More
// slices put more wavefronts on each SIMD for the same tile, which hides the
// dependent-MFMA and LDS latencies of a tile grid too small to fill the GPU
// otherwise, without a second kernel or workspace.  DEPTH 2 issues each
// stage's global loads two K steps ahead (for tiles whose K step is shorter
// than the memory latency).
template <int BM_, int BN_, int BK_, int WAVES_M_, int WAVES_N_, int UNROLL_ = BK_ / 2,
          int GROUP_M_ = 8, bool PRIO_ = false, int KSLICE_ = 1, int DEPTH_ = 1, int MS_ = 32,
          bool EARLY_ = false>
struct MfmaTile {
  static constexpr int BM = BM_, BN = BN_, BK = BK_;
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  static constexpr int KSLICE = KSLICE_;
  static constexpr int THREADS = 64 * WAVES_M * WAVES_N * KSLICE;
  static constexpr int UNROLL = UNROLL_;
  static constexpr int GROUP_M = GROUP_M_;
  static constexpr bool PRIO = PRIO_;
  // Prefetch depth: global loads of a stage are issued DEPTH K steps before
  // it is computed (2 = two register sets alternating).
  static constexpr int DEPTH = DEPTH_;
  static_assert(DEPTH == 1 || DEPTH == 2, "prefetch depth 1 or 2");
  // Matrix instruction: 32 x 32 x 2 or 16 x 16 x 4 blocks.
  static constexpr int MS = MS_;
  // With DEPTH 1: store the next stage into LDS before this stage's MFMAs
  // (and load the one after) rather than after them.
  static constexpr bool EARLY = EARLY_;
};

template <int N>
struct VecT;
template <>
struct VecT<1> { typedef float type; };
template <>
struct VecT<2> { typedef float2 type; };
template <>
struct VecT<4> { typedef float4 type; };

template <int N>
__device__ __forceinline__ float vget(const typename VecT<N>::type& v, int i);
template <>
__device__ __forceinline__ float vget<1>(const float& v, int) { return v; }
template <>
__device__ __forceinline__ float vget<2>(const float2& v, int i) {
  return i == 0 ? v.x : v.y;
}
template <>
__device__ __forceinline__ float vget<4>(const float4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// MODE kWhole: the host guarantees M % BM == N % BN == K % BK == 0, so every
// tile and K step is whole and the kernel carries no bounds logic (fewer
// registers and instructions).  kRaggedK: whole M and N tiles, K not a
// multiple of BK; only the last K step masks (k beyond K reads as zero), and
// the register budget stays that of kWhole, so two blocks of the 256 x 128
// tile still share a CU.  kEdge handles any shape.
constexpr int kWhole = 0, kRaggedK = 1, kEdge = 2;

// One operand panel's share of a K step for one thread: E (= BM or BN) rows
// or columns of the panel by BK values of k, moved from global memory into
// the k-major LDS array X[k][e] as float4 groups, THREADS threads, ITERS
// groups each.  KCONTIG: the source has k contiguous (row-major A, a
// transposed B stored N x K): group = 4 consecutive k of one e, transposed on
// the way into LDS.  Otherwise e is contiguous (row-major B, a transposed A
// stored K x M): group = 4 consecutive e of one k, copied as is.  Groups
// outside the matrix (e beyond its extent, k beyond K) read as zero and are
// never dereferenced.
template <int E, int BK, int THREADS, bool KCONTIG>
struct Panel {
  static constexpr int ITERS = (E * BK / 4) / THREADS;
  static_assert(ITERS >= 1 && ITERS * THREADS * 4 == E * BK, "panel not evenly staged");
  const float* ptr[ITERS];
  float4 reg[2][ITERS];  // set 1 only with prefetch depth 2

  // group index of (thread, s) -> (e, k) inside the panel
  // A lane quad takes the BK/4 groups of one e (a row's 64 contiguous bytes
  // at BK = 16) with KCONTIG, or 16 consecutive e of one k otherwise.
  __device__ static int e_of(int idx) { return KCONTIG ? idx / (BK / 4) : 4 * (idx % (E / 4)); }
  __device__ static int k_of(int idx) { return KCONTIG ? 4 * (idx % (BK / 4)) : idx / (E / 4); }

  // LDS layout: X[k / 4][(k % 4) * E + e] -- unpadded k-rows, groups of
  // four k-rows GROUP words apart.  Measured on MI355X (bank-conflict
  // counter over single access patterns): a 128-bit read whose 16-lane
  // groups each cover 256 contiguous bytes of one row -- the fragment reads
  // -- is conflict-free when the row stride is a multiple of 256 bytes and
  // takes 4 extra cycles otherwise, and 32-bit writes are served as two
  // half-wavefronts on 32 banks.  An MFMA step reads k-rows of one group
  // (row stride 4E bytes, E a multiple of 64): conflict-free.  The
  // transposing store (KCONTIG) has a half-wavefront write the BK/4 k-groups
  // of 128/BK consecutive e; groups 128/BK words apart put those writes on
  // 32 different banks.
  static constexpr int GROUP = 4 * E + (KCONTIG ? 128 / BK : 0);
  static_assert(E % 64 == 0 && GROUP % 4 == 0, "rows of 64-word multiples, 16-byte aligned groups");

  __device__ void init(const float* base, int64_t ld, int64_t e0, int64_t k_lo, int tid) {
#pragma unroll
    for (int s = 0; s < ITERS; ++s) {
      const int idx = tid + s * THREADS;
      ptr[s] = KCONTIG ? base + (e0 + e_of(idx)) * ld + k_lo + k_of(idx)
                       : base + (k_lo + k_of(idx)) * ld + e0 + e_of(idx);
    }
  }
  // whole K step, whole tile (load_one: group s only)
  template <int W>
  __device__ void load_one(int s, int64_t k0, int64_t ld) {
    reg[W][s] = ld_global4(ptr[s] + (KCONTIG ? k0 : k0 * ld));
  }
  template <int W>
  __device__ void load_whole(int64_t k0, int64_t ld) {
#pragma unroll
    for (int s = 0; s < ITERS; ++s) load_one<W>(s, k0, ld);
  }
  // last K step of a whole tile: k at or beyond K reads as zero
  template <int W>
  __device__ void load_ragged_k(int64_t k0, int64_t K, int64_t ld, int tid) {
#pragma unroll
    for (int s = 0; s < ITERS; ++s) {
      const int64_t k = k0 + k_of(tid + s * THREADS);
      if (KCONTIG) {
        const float* q = ptr[s] + k0;
        reg[W][s] = make_float4(k < K ? q[0] : 0.0f, k + 1 < K ? q[1] : 0.0f,
                                k + 2 < K ? q[2] : 0.0f, k + 3 < K ? q[3] : 0.0f);
      } else {
        reg[W][s] = k < K ? ld_global4(ptr[s] + k0 * ld) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      }
    }
  }
  // any K step of any tile: e0 is the tile's first row/column, ext the
  // matrix's extent in e (M or N)
  template <int W>
  __device__ void load_edge(int64_t k0, int64_t K, int64_t ld, int64_t e0, int64_t ext,
                            int tid) {
#pragma unroll
    for (int s = 0; s < ITERS; ++s) {
      const int idx = tid + s * THREADS;
      const int64_t e = e0 + e_of(idx), k = k0 + k_of(idx);
      if (KCONTIG)
        reg[W][s] = load4(ptr[s] - k_of(idx), k, K, e < ext);
      else
        reg[W][s] = load4(ptr[s] + k0 * ld - e, e, ext, k < K);
    }
  }
  // group s of register set W into the LDS stage X (store_one), or all of them
  template <int W>
  __device__ void store_one(int s, float (*X)[GROUP], int tid) const {
    const int idx = tid + s * THREADS;
    const int e = e_of(idx), k = k_of(idx);
    float* const g = X[k / 4];
    if (KCONTIG) {  // k % 4 == 0: the group's four rows
      g[0 * E + e] = reg[W][s].x;
      g[1 * E + e] = reg[W][s].y;
      g[2 * E + e] = reg[W][s].z;
      g[3 * E + e] = reg[W][s].w;
    } else {
      *reinterpret_cast<float4*>(&g[(k % 4) * E + e]) = reg[W][s];
    }
  }
  template <int W>
  __device__ void store(float (*X)[GROUP], int tid) const {
#pragma unroll
    for (int s = 0; s < ITERS; ++s) store_one<W>(s, X, tid);
  }
};
//
// SPLIT (split K): work item t is K slice t / ntiles, k in
// [k_lo, k_lo + k_split), of tile t % ntiles; it stores its raw float32 sums
// (no alpha, beta or C) into plane t / ntiles of ws, an M x N row-major array
// per slice, and k_splitk_reduce adds the planes in slice order.  The slice
// length is a multiple of BK, so every slice but the last is whole.
//
// TA / TB: A is given transposed (stored K x M, row stride lda >= M) / B is
// given transposed (stored N x K, ldb >= K); C is always M x N row-major.
template <class T, int MODE, bool SPLIT = false, bool TA = false, bool TB = false>
__global__ __launch_bounds__(T::THREADS) void k_level9(Problem p, int64_t tiles_m,
                                                       int64_t tiles_n, int64_t ntiles,
                                                       int64_t k_split,
                                                       float* __restrict__ ws) {
  constexpr int BM = T::BM, BN = T::BN, BK = T::BK, THREADS = T::THREADS;
  constexpr int WTM = BM / T::WAVES_M, WTN = BN / T::WAVES_N;
  typedef MfmaOp<T::MS> Op;
  constexpr int DIM = Op::DIM, KPER = Op::KPER, REGS = Op::REGS;
  constexpr int BLK_M = WTM / DIM, BLK_N = WTN / DIM;
  typedef Panel<BM, BK, THREADS, !TA> PanelA;
  typedef Panel<BN, BK, THREADS, TB> PanelB;
  constexpr int GA = PanelA::GROUP, GB = PanelB::GROUP;
  static_assert(BLK_M * DIM == WTM && BLK_N * DIM == WTN, "wave tile not whole blocks");
  static_assert(BK % KPER == 0, "a stage is whole MFMA steps");
  static_assert((BK / KPER) % T::KSLICE == 0, "K slices must split a stage's MFMA steps evenly");
  constexpr int WAVE_TILES = T::WAVES_M * T::WAVES_N;
  constexpr int STEPS = BK / KPER / T::KSLICE;         // MFMA steps per stage per wavefront
  constexpr int PER_WAVE = BLK_M * BLK_N * REGS * 64;  // accumulator floats per wavefront
  typedef typename VecT<BLK_M>::type AFrag;
  typedef typename VecT<BLK_N>::type BFrag;

  // LDS: the two stages of A and B; with K slices, the slices' sums meet in
  // the same memory once the K loop is over (the stages are free then).
  constexpr int STAGE_FLOATS = 2 * (BK / 4) * (GA + GB);
  constexpr int RED_FLOATS = (T::KSLICE - 1) * WAVE_TILES * PER_WAVE;
  __shared__ __align__(16) float smem[STAGE_FLOATS > RED_FLOATS ? STAGE_FLOATS : RED_FLOATS];
  float (*const As)[BK / 4][GA] = reinterpret_cast<float (*)[BK / 4][GA]>(smem);
  float (*const Bs)[BK / 4][GB] = reinterpret_cast<float (*)[BK / 4][GB]>(smem + 2 * (BK / 4) * GA);
  float* const red = smem;

  const int tid = threadIdx.x;
  const int wave = tid / 64, lane = tid % 64;
  const int kslice = wave / WAVE_TILES, wv = wave % WAVE_TILES;
  const int wm = wv / T::WAVES_N, wn = wv % T::WAVES_N;
  const int lrow = lane % DIM, kg = lane / DIM;  // block row/column, k within a step
  // LDS offsets (words) of this lane's fragments inside one k-row
  const int a_off = wm * WTM + BLK_M * lrow;
  const int b_off = wn * WTN + BLK_N * lrow;

  const int64_t items = SPLIT ? ntiles * ceil_div(p.K, k_split) : ntiles;
  const int64_t first = xcd_contiguous(blockIdx.x, gridDim.x);
  for (int64_t item = first; item < items; item += gridDim.x) {
    const int64_t t = SPLIT ? item % ntiles : item;
    const int64_t split = SPLIT ? item / ntiles : 0;
    const int64_t k_lo = split * k_split;
    const int64_t K = SPLIT ? (p.K - k_lo < k_split ? p.K - k_lo : k_split) : p.K;
    const int64_t nk = ceil_div(K, BK);
    const int64_t group = T::GROUP_M * tiles_n;
    const int64_t first_m = (t / group) * T::GROUP_M;
    const int64_t gm = tiles_m - first_m < T::GROUP_M ? tiles_m - first_m : T::GROUP_M;
    const int64_t in = t % group;
    const int64_t row0 = (first_m + in % gm) * BM;
    const int64_t col0 = (in / gm) * BN;

    typename Op::acc_t acc[BLK_M][BLK_N];
#pragma unroll
    for (int bi = 0; bi < BLK_M; ++bi)
#pragma unroll
      for (int bj = 0; bj < BLK_N; ++bj)
#pragma unroll
        for (int r = 0; r < REGS; ++r) acc[bi][bj][r] = 0.0f;

    // This thread's share of the A and B panels of each K step (rows of A
    // beyond M, columns of B beyond N and k beyond K read as zero).
    const bool interior = MODE != kEdge || (row0 + BM <= p.M && col0 + BN <= p.N);
    PanelA pa;
    PanelB pb;
    pa.init(p.A, p.lda, row0, k_lo, tid);
    pb.init(p.B, p.ldb, col0, k_lo, tid);
    // load<W>: stage at k0 into register set W; store<W>: set W into LDS
    // stage buffer W' (W' = W with depth 2, the alternating buffer with 1).
    typedef std::integral_constant<int, 0> Set0;
    typedef std::integral_constant<int, 1> Set1;
    auto load = [&](auto set, int64_t k0) {
      constexpr int W = decltype(set)::value;
      if (MODE == kWhole || (interior && k0 + BK <= K)) {
        // whole K step inside the matrix: no bounds tests (uniform branch)
        pa.template load_whole<W>(k0, p.lda);
        pb.template load_whole<W>(k0, p.ldb);
      } else if (MODE == kRaggedK) {
        pa.template load_ragged_k<W>(k0, K, p.lda, tid);
        pb.template load_ragged_k<W>(k0, K, p.ldb, tid);
      } else {
        pa.template load_edge<W>(k0, K, p.lda, row0, p.M, tid);
        pb.template load_edge<W>(k0, K, p.ldb, col0, p.N, tid);
      }
    };
    auto store = [&](auto set, int buf) {
      constexpr int W = decltype(set)::value;
      pa.template store<W>(As[buf], tid);
      pb.template store<W>(Bs[buf], tid);
    };
    // The MFMA steps of one stage.  PRIO: two blocks share each CU's matrix
    // pipes and a block is only as fast as its slowest wavefront at the
    // barrier, so a wavefront takes priority 1 while it issues MFMAs (and 3
    // while it stores the next stage and waits at the barrier, below: the
    // stragglers reach the barrier sooner), then drops to 0.  Measured on
    // MI355X: +3 % at 4096^3 with 256 x 128 tiles.
    auto mfma_stage = [&](int cur) {
      if (T::PRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll T::UNROLL
      for (int s = 0; s < STEPS; ++s) {
        // (the KPER k-rows k0 + kg of one MFMA step lie in one group)
        const int k0 = KPER * (kslice * STEPS + s), r = k0 % 4 + kg;
        const AFrag af = *reinterpret_cast<const AFrag*>(&As[cur][k0 / 4][r * BM + a_off]);
        const BFrag bf = *reinterpret_cast<const BFrag*>(&Bs[cur][k0 / 4][r * BN + b_off]);
#pragma unroll
        for (int bi = 0; bi < BLK_M; ++bi)
#pragma unroll
          for (int bj = 0; bj < BLK_N; ++bj)
            acc[bi][bj] = Op::mma(vget<BLK_M>(af, bi), vget<BLK_N>(bf, bj), acc[bi][bj]);
      }
      if (T::PRIO) __builtin_amdgcn_s_setprio(3);
    };
    auto barrier = [&]() {
      __syncthreads();
      if (T::PRIO) __builtin_amdgcn_s_setprio(0);
    };

    if (T::DEPTH == 1 && T::EARLY) {
      // Stage kt + 1 goes from registers into LDS before stage kt's MFMAs
      // (its buffer was released by the previous barrier) and the registers
      // take stage kt + 2 right after: the stores' latency hides under the
      // MFMAs instead of preceding the barrier.
      load(Set0(), 0);
      store(Set0(), 0);
      if (nk > 1) load(Set0(), BK);
      __syncthreads();
      for (int64_t kt = 0; kt < nk; ++kt) {
        const int cur = static_cast<int>(kt & 1);
        if (kt + 1 < nk) store(Set0(), cur ^ 1);
        if (kt + 2 < nk) load(Set0(), (kt + 2) * BK);
        mfma_stage(cur);
        barrier();
      }
    } else if (T::DEPTH == 1) {
      load(Set0(), 0);
      store(Set0(), 0);
      __syncthreads();
      for (int64_t kt = 0; kt < nk; ++kt) {
        const int cur = static_cast<int>(kt & 1);
        const bool more = kt + 1 < nk;
        if (more) load(Set0(), (kt + 1) * BK);
        mfma_stage(cur);
        if (more) store(Set0(), cur ^ 1);
        barrier();
      }
    } else {
      // Stage j lives in register set j % 2 and LDS buffer j % 2; its loads
      // are issued at the start of step j - 2 and stored at the end of step
      // j - 1, after the buffer's previous stage (j - 2) has been read.
      load(Set0(), 0);
      store(Set0(), 0);
      if (nk > 1) load(Set1(), BK);
      __syncthreads();
      for (int64_t kt = 0; kt < nk; kt += 2) {
        if (kt + 2 < nk) load(Set0(), (kt + 2) * BK);
        mfma_stage(0);
        if (kt + 1 < nk) store(Set1(), 1);
        barrier();
        if (kt + 1 >= nk) break;
        if (kt + 3 < nk) load(Set1(), (kt + 3) * BK);
        mfma_stage(1);
        if (kt + 2 < nk) store(Set0(), 0);
        barrier();
      }
    }

    if (T::KSLICE > 1) {
      // Slices 1.. hand their sums to slice 0 through LDS (lane-contiguous,
      // conflict free; the K loop's last barrier has freed the stages that
      // red overlays); slice 0 adds them in slice order and runs the
      // epilogue.  The second barrier frees red before the next tile stages.
      if (kslice > 0) {
        float* dst = red + ((kslice - 1) * WAVE_TILES + wv) * PER_WAVE + lane;
#pragma unroll
        for (int bi = 0; bi < BLK_M; ++bi)
#pragma unroll
          for (int bj = 0; bj < BLK_N; ++bj)
#pragma unroll
            for (int r = 0; r < REGS; ++r) dst[((bi * BLK_N + bj) * REGS + r) * 64] = acc[bi][bj][r];
      }
      __syncthreads();
      if (kslice == 0) {
#pragma unroll
        for (int ks = 1; ks < T::KSLICE; ++ks) {
          const float* src = red + ((ks - 1) * WAVE_TILES + wv) * PER_WAVE + lane;
#pragma unroll
          for (int bi = 0; bi < BLK_M; ++bi)
#pragma unroll
            for (int bj = 0; bj < BLK_N; ++bj)
#pragma unroll
              for (int r = 0; r < REGS; ++r) acc[bi][bj][r] += src[((bi * BLK_N + bj) * REGS + r) * 64];
        }
      }
      __syncthreads();
      if (kslice > 0) continue;
    }

    // Epilogue: register r of block (bi, bj) is C[row(bi, r)][col(bj)]; a
    // lane's BLK_N outputs of one row are adjacent.
    // Each lane keeps one base pointer per block row; the offsets of its 16
    // registers' rows are lane-independent multiples of ldc (scalar work).
    const int64_t col = col0 + b_off;
    const bool vec_ok = MODE != kEdge || (BLK_N > 1 && col + BLK_N - 1 < p.N);
    if (SPLIT) {
      // raw sums into this slice's plane (row stride N)
      float* const plane = ws + split * int64_t(p.M) * p.N;
#pragma unroll
      for (int bi = 0; bi < BLK_M; ++bi) {
        const int64_t row_base = row0 + wm * WTM + BLK_M * Op::row(kg, 0) + bi;
        float* const w_base = plane + row_base * p.N + col;
#pragma unroll
        for (int r = 0; r < REGS; ++r) {
          const int dr = BLK_M * (Op::row(kg, r) - Op::row(kg, 0));
          if (!interior && row_base + dr >= p.M) continue;
          float* w = w_base + dr * p.N;
          float o[BLK_N];
#pragma unroll
          for (int bj = 0; bj < BLK_N; ++bj) o[bj] = acc[bi][bj][r];
          if (interior || vec_ok) {
            __builtin_memcpy(w, o, sizeof(o));
          } else {
#pragma unroll
            for (int bj = 0; bj < BLK_N; ++bj)
              if (col + bj < p.N) w[bj] = o[bj];
          }
        }
      }
      continue;
    }
#pragma unroll
    for (int bi = 0; bi < BLK_M; ++bi) {
      const int64_t row_base = row0 + wm * WTM + BLK_M * Op::row(kg, 0) + bi;
      float* const c_base = p.C + row_base * p.ldc + col;
      auto row_in = [&](int r) {
        return interior || row_base + BLK_M * (Op::row(kg, r) - Op::row(kg, 0)) < p.M;
      };
      auto c_row = [&](int r) { return c_base + BLK_M * (Op::row(kg, r) - Op::row(kg, 0)) * p.ldc; };
      if (interior || vec_ok) {
        // One 64- or 128-bit access per lane and row (4-byte alignment
        // suffices).  With beta != 0 the old values of four rows are loaded
        // before their stores: the compiler cannot move a load of C above a
        // store to C (it cannot tell the rows apart), so loads interleaved
        // with stores would each wait out a full memory latency (four rows
        // at a time bounds the registers this takes).
        if (p.beta != 0.0f) {
          constexpr int RB = REGS < 4 ? REGS : 4;
#pragma unroll
          for (int r0 = 0; r0 < REGS; r0 += RB) {
            float old[RB][BLK_N];
#pragma unroll
            for (int r = r0; r < r0 + RB; ++r)
              if (row_in(r)) __builtin_memcpy(old[r - r0], c_row(r), sizeof(old[0]));
#pragma unroll
            for (int r = r0; r < r0 + RB; ++r) {
              if (!row_in(r)) continue;
              float o[BLK_N];
#pragma unroll
              for (int bj = 0; bj < BLK_N; ++bj)
                o[bj] = fmaf(p.beta, old[r - r0][bj], p.alpha * acc[bi][bj][r]);
              __builtin_memcpy(c_row(r), o, sizeof(o));
            }
          }
        } else {
#pragma unroll
          for (int r = 0; r < REGS; ++r) {
            if (!row_in(r)) continue;
            float o[BLK_N];
#pragma unroll
            for (int bj = 0; bj < BLK_N; ++bj) o[bj] = p.alpha * acc[bi][bj][r];
            __builtin_memcpy(c_row(r), o, sizeof(o));
          }
        }
      } else {
#pragma unroll
        for (int r = 0; r < REGS; ++r) {
          if (!row_in(r)) continue;
          float* c = c_row(r);
#pragma unroll
          for (int bj = 0; bj < BLK_N; ++bj)
            if (col + bj < p.N)
              c[bj] = epilogue(acc[bi][bj][r], p.alpha, p.beta, c + bj);
        }
      }
    }
  }
}

template <class T>
Geometry tile_geometry(int M, int N, int K) {
  return make_geometry(M, N, K, T::BM, T::BN, T::BK, T::THREADS);
}

template <class T, bool TA = false, bool TB = false>
hipError_t launch_tiles(const Problem& p, hipStream_t s) {
  const Geometry g = tile_geometry<T>(p.M, p.N, p.K);
  const dim3 grid(static_cast<unsigned>(g.workgroups)), block(T::THREADS);
  const int64_t tm = ceil_div(p.M, T::BM), tn = ceil_div(p.N, T::BN);
  const bool whole_mn = p.M % T::BM == 0 && p.N % T::BN == 0;
  if (whole_mn && p.K % T::BK == 0)
    hipLaunchKernelGGL((k_level9<T, kWhole, false, TA, TB>), grid, block, 0, s, p, tm, tn,
                       g.tiles, int64_t(p.K), nullptr);
  else if (whole_mn)
    hipLaunchKernelGGL((k_level9<T, kRaggedK, false, TA, TB>), grid, block, 0, s, p, tm, tn,
                       g.tiles, int64_t(p.K), nullptr);
  else
    hipLaunchKernelGGL((k_level9<T, kEdge, false, TA, TB>), grid, block, 0, s, p, tm, tn,
                       g.tiles, int64_t(p.K), nullptr);
  return hipGetLastError();
}

// Split K: ceil(K / k_split) slices per tile (k_split a multiple of BK),
// raw sums into ws (slices x M x N floats).
template <class T>
Geometry split_geometry(int M, int N, int K, int64_t k_split) {
  Geometry g = make_geometry(M, N, K, T::BM, T::BN, T::BK, T::THREADS);
  g.tiles *= ceil_div(K, k_split);
  const int64_t cap = kMaxWorkItems / T::THREADS;
  g.workgroups = g.tiles < cap ? g.tiles : cap;
  g.k_steps = ceil_div(k_split, T::BK);
  return g;
}

template <class T, bool TA = false, bool TB = false>
hipError_t launch_split(const Problem& p, int64_t k_split, float* ws, hipStream_t s) {
  const Geometry g = split_geometry<T>(p.M, p.N, p.K, k_split);
  const dim3 grid(static_cast<unsigned>(g.workgroups)), block(T::THREADS);
  const int64_t tm = ceil_div(p.M, T::BM), tn = ceil_div(p.N, T::BN);
  const bool whole_mn = p.M % T::BM == 0 && p.N % T::BN == 0;
  if (whole_mn && p.K % T::BK == 0)
    hipLaunchKernelGGL((k_level9<T, kWhole, true, TA, TB>), grid, block, 0, s, p, tm, tn,
                       tm * tn, k_split, ws);
  else if (whole_mn)
    hipLaunchKernelGGL((k_level9<T, kRaggedK, true, TA, TB>), grid, block, 0, s, p, tm, tn,
                       tm * tn, k_split, ws);
  else
    hipLaunchKernelGGL((k_level9<T, kEdge, true, TA, TB>), grid, block, 0, s, p, tm, tn,
                       tm * tn, k_split, ws);
  return hipGetLastError();
}

// The tile shapes the level uses, chosen per problem from measurements on
// MI355X (256 CUs).  Whole-tile problems large enough to give every CU two
// 256 x 128 tiles take the big tile (fewest L2->LDS bytes per FLOP, 8
// wavefronts per block); mid-size whole-tile problems take 128 x 128 with
// 32-deep K steps; large ragged problems (4097^3 leaves a one-row /
// one-column fringe of tiles) take 128 x 64, whose many small blocks soak up
// the fringe; small problems take 64 x 64 so that more CUs get work.
// The big tile runs 16 x 16 x 4 blocks: each wavefront's 64 x 64 wave tile is
// 4 x 4 blocks, 16 independent accumulator chains of 8-pass instructions
// (against 4 chains of 16-pass ones with 32 x 32 blocks); measured on
// MI355X: 138.2 against 136.6 TFLOP/s at 4096^3, 131.8 against 128.2 at
// 4097^3.  (The 16 x 16 form of the other tiles measured equal or slower.)
typedef MfmaTile<256, 128, 16, 4, 2, 4, 8, true, 1, 1, 16> TileHuge;
typedef MfmaTile<128, 128, 32, 4, 1, 16, 8, true> TileLarge;
typedef MfmaTile<128, 64, 16, 2, 2> TileMid;
typedef MfmaTile<64, 64, 16, 2, 2> TileSmall;
// Two K slices per stage (8 wavefronts): for tile grids of about one block
// per CU, where a single wavefront per SIMD leaves MFMA and LDS latency
// exposed.  Measured on MI355X: 64 x 64 at 1024^3 +18 %, at 3072^3 +10 %;
// 128 x 128 (2 x 2 wave tiles of 64 x 64) at 2048^3 +5 %.  The 64 x 64 tile
// also prefetches two K steps ahead with raised priority around the barrier
// (its 32-deep K step is shorter than a global load's latency): +3-4 % at
// 768^3-3072^3; the 128 x 128 one loses 4 % with it and keeps one step.
typedef MfmaTile<128, 128, 32, 2, 2, 16, 8, false, 2> TileLargeSliced;
// The 128 x 128 tile as split-K work items (K slices of 256 to 1024) stores
// each stage into LDS before the previous stage's MFMAs: measured on MI355X
// +5.9 % at 1024 x 1024 x 4096 and +4 % at 1024 x 1024 x 8192, where it
// costs the unsplit tile 1.6 % (2048 x 4096 x 2048) and the 256 x 128 tile
// 1.5-3 %.
typedef MfmaTile<128, 128, 32, 4, 1, 16, 8, true, 1, 1, 32, true> TileLargeSplit;
typedef MfmaTile<64, 64, 32, 2, 2, 16, 8, true, 2, 2> TileSmallSliced;
constexpr int kCUs = 256;

// Launch a tile shape on a problem (MODE chosen from the problem's shape).
template <bool TA, bool TB>
hipError_t launch_shape_t(Shape shape, const Problem& p, hipStream_t s) {
  switch (shape) {
    case Shape::kHuge: return launch_tiles<TileHuge, TA, TB>(p, s);
    case Shape::kLarge: return launch_tiles<TileLarge, TA, TB>(p, s);
    case Shape::kMid: return launch_tiles<TileMid, TA, TB>(p, s);
    case Shape::kLargeSliced: return launch_tiles<TileLargeSliced, TA, TB>(p, s);
    case Shape::kSmallSliced: return launch_tiles<TileSmallSliced, TA, TB>(p, s);
    default: return launch_tiles<TileSmall, TA, TB>(p, s);
  }
}

// The same with K split into slices of k_split (raw sums into ws).
template <bool TA, bool TB>
hipError_t launch_split_shape_t(Shape shape, const Problem& p, int64_t k_split, float* ws,
                                hipStream_t s) {
  switch (shape) {
    case Shape::kHuge: return launch_split<TileHuge, TA, TB>(p, k_split, ws, s);
    case Shape::kLarge: return launch_split<TileLargeSplit, TA, TB>(p, k_split, ws, s);
    case Shape::kMid: return launch_split<TileMid, TA, TB>(p, k_split, ws, s);
    case Shape::kLargeSliced: return launch_split<TileLargeSliced, TA, TB>(p, k_split, ws, s);
    case Shape::kSmallSliced: return launch_split<TileSmallSliced, TA, TB>(p, k_split, ws, s);
    default: return launch_split<TileSmall, TA, TB>(p, k_split, ws, s);
  }
}

}  // namespace
}  // namespace sgemm
