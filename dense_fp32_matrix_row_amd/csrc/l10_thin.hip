// l10_thin.hip -- the thin-problem kernels of the dispatching rung: C blocks
// with at most kThin (16) rows or at most kThin columns.
//
// A thin product reads one operand in full and does little arithmetic per
// byte (M = 1 is a matrix-vector product), so it is HBM-bound; a matrix-core
// tile would leave most of its 32 x 32 blocks empty.  The pages' answer for
// a row panel is one lane per output column with the K loop inside ([SIX]
// K1-K2); a single M = 1 row of 4097 columns gives only 4097 lanes, far from
// filling 256 CUs, so here each output's K sum is split over the lanes and
// wavefronts of one block instead and combined in a fixed order:
//   - per lane, a float32 FMA chain over its own k values (ascending);
//   - across lanes, an xor butterfly (partner order fixed by lane bits);
//   - across wavefronts, an in-order sum through LDS.
// The order depends only on the shape, never on timing: results are
// bit-reproducible, with no atomics and no workspace.
//
// Two forms: vector-ALU FMA chains (below, for one to four rows or
// columns of short problems), and a matrix-core form for the rest, whose
// 16-row MFMA block takes up to sixteen rows at once (further below).
//
// Used for problems with M <= 16 or N <= 16, and for the one- to
// sixteen-row/column fringe left beside the matrix-core tiles of large
// ragged problems (4097^3: a 4096 x 4096 tile grid plus a 1-row and a
// 1-column fringe).
#include "sgemm_internal.h"

namespace sgemm {
namespace {

__device__ __forceinline__ float fget(const float4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// The vector-ALU kernels walk K in two loops: the steps whose loads all lie
// inside the operands for the whole block (a block-uniform test) take
// 128-bit loads with no per-lane test, issued back to back; the step at the
// end of K, and every step of a block at the right edge, load through
// load4's per-lane checks, behind which the compiler makes each load wait
// for the one before (the many wavefronts per CU hide most of that).  Same
// results; 4097 x 1 x 4097 22.8 -> 21.0 us, 4 x 4096 x 4096 with B stored
// transposed 18.6 -> 17.0.  Edge steps without the per-lane checks
// (addresses clamped into the operand, zeros past K) needed up to 80 % more
// registers and lost wavefronts per CU (4097 x 1 x 4097: 37 us), and the
// same split in the matrix-core kernel below was slower on half the shapes
// tried (16 x 8192 x 8192: 62 -> 66-102 us), so that kernel keeps one loop.

// ---------------------------------------------------------------------------
// Few rows: M <= RP.  Block b owns columns [16b, 16b + 16).  Lane l of
// wavefront w takes the column quad q = l % 4 (4 adjacent columns, one
// 128-bit B access) and, in each sweep of 64*WAVES k values, the k quad
// g = l / 4 of its wavefront's 64: k = sweep*64*WAVES + 64*w + 4*g .. +3.
// For each such k it reads 4 B rows (4 x 4 floats) and the RP A values of
// those k (one 128-bit access per row of A).
template <int RP>
struct FewRows {
  static_assert(RP <= 4, "more rows go to the matrix-core form");
  static constexpr int WAVES = 16;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int KSWEEP = 64 * WAVES;
};

// One lane's k quad k .. k + 3 of a sweep: its loads, then its FMAs (two
// copies, so that the 128-bit form's loads issue back to back).  FULL: the
// block's 16 columns and every lane's k quad are inside B and A.
template <int RP, bool TA, bool TB, bool FULL>
__device__ __forceinline__ void rows_step(const Problem& p, int64_t k, int64_t col, float (&acc)[RP][4]) {
  float4 b[4], a[RP];
  if (TB) {
    float4 v[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
      v[c] = FULL ? ld_global4(p.B + (col + c) * p.ldb + k) : load4(p.B + (col + c) * p.ldb, k, p.K, col + c < p.N);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      b[j] = make_float4(fget(v[0], j), fget(v[1], j), fget(v[2], j), fget(v[3], j));
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      b[j] = FULL ? ld_global4(p.B + (k + j) * p.ldb + col) : load4(p.B + (k + j) * p.ldb, col, p.N, k + j < p.K);
  }
#pragma unroll
  for (int r = 0; r < RP; ++r) {
    if (TA) {
      const bool ok = r < p.M;  // uniform
      const float* at = p.A + k * p.lda + r;
      a[r] = FULL ? make_float4(ok ? at[0] : 0.0f, ok ? at[p.lda] : 0.0f, ok ? at[2 * p.lda] : 0.0f,
                                ok ? at[3 * p.lda] : 0.0f)
                  : make_float4(ok && k < p.K ? at[0] : 0.0f, ok && k + 1 < p.K ? at[p.lda] : 0.0f,
                                ok && k + 2 < p.K ? at[2 * p.lda] : 0.0f, ok && k + 3 < p.K ? at[3 * p.lda] : 0.0f);
    } else {
      a[r] = FULL && r < p.M ? ld_global4(p.A + r * p.lda + k) : load4(p.A + r * p.lda, k, p.K, r < p.M);
    }
  }
#pragma unroll
  for (int r = 0; r < RP; ++r) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float av = fget(a[r], j);
      acc[r][0] = fmaf(av, b[j].x, acc[r][0]);
      acc[r][1] = fmaf(av, b[j].y, acc[r][1]);
      acc[r][2] = fmaf(av, b[j].z, acc[r][2]);
      acc[r][3] = fmaf(av, b[j].w, acc[r][3]);
    }
  }
}

// TA: A stored K x M (element (r, k) at A[k * lda + r]); TB: B stored N x K
// (element (k, n) at B[n * ldb + k]: the lane's four columns come as four
// 128-bit reads along k and are transposed in registers).
template <int RP, bool TA, bool TB>
__global__ __launch_bounds__(FewRows<RP>::THREADS) void k_few_rows(Problem p,
                                                                   int64_t nblocks) {
  constexpr int WAVES = FewRows<RP>::WAVES, KSWEEP = FewRows<RP>::KSWEEP;
  __shared__ float red[WAVES][RP][16];
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
  const int q = lane % 4, g = lane / 4;

  // neighbouring column blocks read the two halves of the same 128-byte B
  // lines: keep them on one XCD (one L2)
  for (int64_t blk = xcd_contiguous(blockIdx.x, gridDim.x); blk < nblocks; blk += gridDim.x) {
    const int64_t c0 = blk * 16;
    const int64_t col = c0 + 4 * q;
    float acc[RP][4];
#pragma unroll
    for (int r = 0; r < RP; ++r)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[r][c] = 0.0f;

    const bool cols_full = c0 + 16 <= p.N;  // block-uniform
    // whole sweeps first (128-bit loads), then the partial sweep at the end
    // of K, and every sweep of a block at the right edge, element by element
    const int64_t k_whole = cols_full ? p.K / KSWEEP * KSWEEP : 0;
    const int64_t k0 = 64 * wave + 4 * g;
    for (int64_t base = 0; base < k_whole; base += KSWEEP) rows_step<RP, TA, TB, true>(p, base + k0, col, acc);
    for (int64_t base = k_whole; base < p.K; base += KSWEEP) rows_step<RP, TA, TB, false>(p, base + k0, col, acc);

    // Sum over the 16 k quads of the wavefront (lane bits 2-5), then over
    // the wavefronts in order.
#pragma unroll
    for (int r = 0; r < RP; ++r)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        float v = acc[r][c];
        v += __shfl_xor(v, 4);
        v += __shfl_xor(v, 8);
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        if (g == 0) red[wave][r][4 * q + c] = v;
      }
    __syncthreads();
    if (tid < RP * 16) {
      const int r = tid / 16, cc = tid % 16;
      float sum = red[0][r][cc];
#pragma unroll
      for (int w = 1; w < WAVES; ++w) sum += red[w][r][cc];
      if (r < p.M && c0 + cc < p.N) {
        float* c = p.C + r * p.ldc + c0 + cc;
        *c = epilogue(sum, p.alpha, p.beta, c);
      }
    }
    __syncthreads();  // red is rewritten by the next column block
  }
}

// ---------------------------------------------------------------------------
// Few columns: N <= WP.  Block b owns rows [16b, 16b + 16), one row per
// wavefront.  K is walked in chunks of KC: the chunk's WP columns of B are
// staged in LDS column by column (Bs[c][k], so that a lane's four k of one
// column are one conflict-free 128-bit read), and lane l takes the k quads
// 4*l + 256*t of the chunk, reading its A row with 128-bit loads (a
// wavefront reads 1 KB of one A row per instruction).  The next chunk's A
// values are requested before the barrier that guards the B staging, so the
// two latencies overlap.
constexpr int kRowsPerBlock = 16;
constexpr int kColThreads = 64 * kRowsPerBlock;

template <int WP>
struct FewCols {
  static_assert(WP <= 4, "more columns go to the matrix-core form");
  static constexpr int KC = 2048;
  static constexpr int QUADS = KC / 256;            // k quads per lane per chunk
};

// TB: B stored N x K (the staged strip is then contiguous along k).  A is
// always row-major here: with A stored K x M a wavefront's row would be a
// strided column, so the dispatcher gives such problems to the tile kernels.
// A chunk's A loads: the lane's QUADS k quads of its wavefront's A row.
// FULL: the chunk lies inside K (128-bit loads, no per-lane test).
template <int WP, bool FULL>
__device__ __forceinline__ void cols_a_loads(const Problem& p, const float* arow, bool has_row, int64_t kc,
                                             int lane, float4 (&a)[FewCols<WP>::QUADS]) {
#pragma unroll
  for (int t = 0; t < FewCols<WP>::QUADS; ++t) {
    const int64_t k = kc + 4 * lane + 256 * t;
    a[t] = FULL ? ld_global4(arow + k) : load4(arow, k, p.K, has_row);
  }
}

template <int WP, bool TB>
__global__ __launch_bounds__(kColThreads) void k_few_cols(Problem p, int64_t nblocks) {
  constexpr int KC = FewCols<WP>::KC, QUADS = FewCols<WP>::QUADS;
  __shared__ __align__(16) float Bs[WP][KC];
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;

  for (int64_t blk = xcd_contiguous(blockIdx.x, gridDim.x); blk < nblocks; blk += gridDim.x) {
    const int64_t row = blk * kRowsPerBlock + wave;
    const bool has_row = row < p.M;
    const float* arow = p.A + (has_row ? row : 0) * p.lda;
    float acc[WP];
#pragma unroll
    for (int c = 0; c < WP; ++c) acc[c] = 0.0f;

    for (int64_t kc = 0; kc < p.K; kc += KC) {
      float4 a[QUADS];
      if (kc + KC <= p.K) cols_a_loads<WP, true>(p, arow, has_row, kc, lane, a);  // uniform
      else cols_a_loads<WP, false>(p, arow, has_row, kc, lane, a);
      __syncthreads();  // every wavefront is done with the previous chunk
      for (int e = tid; e < WP * KC; e += kColThreads) {
        const int c = e / KC, kk = e % KC;
        const bool ok = kc + kk < p.K && c < p.N;
        Bs[c][kk] = !ok ? 0.0f : TB ? p.B[c * p.ldb + kc + kk] : p.B[(kc + kk) * p.ldb + c];
      }
      __syncthreads();
      if (has_row) {
#pragma unroll
        for (int t = 0; t < QUADS; ++t) {
          const int kk = 4 * lane + 256 * t;
#pragma unroll
          for (int c = 0; c < WP; ++c) {
            const float4 b = *reinterpret_cast<const float4*>(&Bs[c][kk]);
            acc[c] = fmaf(a[t].x, b.x, acc[c]);
            acc[c] = fmaf(a[t].y, b.y, acc[c]);
            acc[c] = fmaf(a[t].z, b.z, acc[c]);
            acc[c] = fmaf(a[t].w, b.w, acc[c]);
          }
        }
      }
    }

    // Sum over the 64 lanes (xor butterfly); lane c then holds column c.
#pragma unroll
    for (int c = 0; c < WP; ++c) {
      float v = acc[c];
      v += __shfl_xor(v, 1);
      v += __shfl_xor(v, 2);
      v += __shfl_xor(v, 4);
      v += __shfl_xor(v, 8);
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 32);
      if (has_row && lane == c && c < p.N) {
        float* cp = p.C + row * p.ldc + c;
        *cp = epilogue(v, p.alpha, p.beta, cp);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Thin problems on the matrix cores.  One form serves both thin shapes:
// C' = alpha * A' * B' + beta * C' with C' at most 16 rows -- C itself for
// few rows, C^T = B^T * A^T for few columns -- where each operand is read
// in its stored orientation:
//   A'[r][k] = TA ? a[k * lda + r] : a[r * lda + k]
//   B'[k][n] = TB ? b[n * ldb + k] : b[k * ldb + n]
//   C'[r][n] = CT ? c[n * ldc + r] : c[r * ldc + n]
// A block owns NB = 16 V columns of C' and all of K.  Its W wavefronts take
// the K groups of 16 in turn; in a group at kb, MFMA step s (0..3) gives
// lane group g = l / 16 the k = kb + 4 g + s, so a lane's four A' values are
// adjacent (one 128-bit read of a row-major A' row) and, when B' is stored
// k-contiguous, so are its four B' values of one column.  v_mfma_f32_16x16x4_f32
// block j takes the columns n0 + V i + j (i = l % 16): with B' row-major a
// lane's V values of one k are adjacent, and the 16 lanes of a k read 16 V
// consecutive floats.  The wavefronts' partial sums meet in LDS and are
// added in wavefront order; nothing depends on timing, and every
// orientation performs the same arithmetic.
struct Thin {
  int M, N, K;  // of C'
  float alpha, beta;
  const float* a;
  int64_t lda;
  const float* b;
  int64_t ldb;
  float* c;
  int64_t ldc;
};

constexpr int kThinWaves = 16;
constexpr int64_t kMaxPanels = 65535;  // grid y limit: panels of 16 rows of C'

template <int V, bool TA, bool TB, bool CT>
__global__ __launch_bounds__(64 * kThinWaves) void k_thin_mfma(Thin whole, int64_t ntiles) {
  typedef float floatx4 __attribute__((ext_vector_type(4)));
  constexpr int W = kThinWaves, NB = 16 * V;
  // blockIdx.y: the panel of 16 rows of C' this block works on (one panel
  // for thin problems; several for small ones, whose 64 x 64 tiles would
  // leave most CUs idle)
  const int64_t panel = blockIdx.y, r0 = 16 * panel;
  Thin t = whole;
  t.M = static_cast<int>(whole.M - r0 < 16 ? whole.M - r0 : 16);
  t.a = TA ? whole.a + r0 : whole.a + r0 * whole.lda;
  t.c = CT ? whole.c + r0 : whole.c + r0 * whole.ldc;
  __shared__ float red[W][16][NB];
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
  const int i = lane % 16, g = lane / 16;
  const bool row_ok = i < t.M;
  for (int64_t tile = xcd_contiguous(blockIdx.x, gridDim.x); tile < ntiles; tile += gridDim.x) {
    const int64_t n0 = tile * NB, nl = n0 + V * i;  // nl: this lane's first column
    floatx4 acc[V];
#pragma unroll
    for (int j = 0; j < V; ++j) acc[j] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    for (int64_t kb = 16 * wave; kb < t.K; kb += 16 * W) {
      const int64_t k = kb + 4 * g;  // steps s = 0..3 take k + s
      float4 av;
      if (TA) {
        av = make_float4(row_ok && k < t.K ? t.a[k * t.lda + i] : 0.0f,
                         row_ok && k + 1 < t.K ? t.a[(k + 1) * t.lda + i] : 0.0f,
                         row_ok && k + 2 < t.K ? t.a[(k + 2) * t.lda + i] : 0.0f,
                         row_ok && k + 3 < t.K ? t.a[(k + 3) * t.lda + i] : 0.0f);
      } else {
        av = load4(t.a + (row_ok ? i : 0) * t.lda, k, t.K, row_ok);
      }
      float bv[4][V];  // [step][column]
      if (TB) {
#pragma unroll
        for (int j = 0; j < V; ++j) {
          const bool ok = nl + j < t.N;
          const float4 v = load4(t.b + (ok ? nl + j : 0) * t.ldb, k, t.K, ok);
#pragma unroll
          for (int s = 0; s < 4; ++s) bv[s][j] = fget(v, s);
        }
      } else {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const bool kok = k + s < t.K;
          const float* row = t.b + (kok ? k + s : 0) * t.ldb;
          if (V == 4) {
            const float4 v = load4(row, nl, t.N, kok);
            bv[s][0] = v.x;
            bv[s][1] = v.y;
            bv[s][2] = v.z;
            bv[s][3] = v.w;
          } else {
#pragma unroll
            for (int j = 0; j < V; ++j) bv[s][j] = kok && nl + j < t.N ? row[nl + j] : 0.0f;
          }
        }
      }
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int j = 0; j < V; ++j)
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(fget(av, s), bv[s][j], acc[j], 0, 0, 0);
    }
    // register r of block j holds C'[4 g + r][n0 + V i + j]
#pragma unroll
    for (int j = 0; j < V; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[wave][4 * g + r][V * i + j] = acc[j][r];
    __syncthreads();
    // consecutive threads take consecutive addresses of C
    for (int e = tid; e < 16 * NB; e += 64 * W) {
      const int r = CT ? e % 16 : e / NB, n = CT ? e / 16 : e % NB;
      float sum = red[0][r][n];
#pragma unroll
      for (int w = 1; w < W; ++w) sum += red[w][r][n];
      if (r < t.M && n0 + n < t.N) {
        float* cp = CT ? t.c + (n0 + n) * t.ldc + r : t.c + r * t.ldc + n0 + n;
        *cp = epilogue(sum, t.alpha, t.beta, cp);
      }
    }
    __syncthreads();  // red is rewritten by the next tile
  }
}

// Columns of C' per lane: the widest (1, 2, 4) that still leaves min_tiles
// tiles; few columns (B' read along k, one 128-bit read per column) stay at
// two at most.  Measured on MI355X (TB/s at 8192 x 8192: 16 rows 4.2-4.6,
// 8 columns 5.7, against 2.4-2.6 on the vector ALUs).
int thin_width(int64_t n, bool few_cols) {
  const int64_t min_tiles = few_cols ? 256 : 512;
  int v = 1;
  while (v < (few_cols ? 2 : 4) && ceil_div(n, 16 * 2 * v) >= min_tiles) v *= 2;
  return v;
}

// The vector-ALU kernels keep one to four rows (columns) of problems below
// 8192 columns (rows), where they measured faster (1 x 4096 x 4096: 4.2
// against 3.8 TB/s).
bool thin_on_valu(int64_t thin, int64_t wide) { return thin <= 4 && wide < 8192; }

template <int V, bool TA, bool TB, bool CT>
hipError_t launch_thin_t(const Thin& t, hipStream_t s) {
  const int64_t ntiles = ceil_div(t.N, 16 * V);
  const int64_t cap = kMaxWorkItems / (64 * kThinWaves);
  const int64_t grid = ntiles < cap ? ntiles : cap;
  const int64_t panels = ceil_div(t.M, 16);
  if (panels > kMaxPanels) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_thin_mfma<V, TA, TB, CT>),
                     dim3(static_cast<unsigned>(grid), static_cast<unsigned>(panels)),
                     dim3(64 * kThinWaves), 0, s, t, ntiles);
  return hipGetLastError();
}

template <bool TA, bool TB, bool CT>
hipError_t launch_thin_op(const Thin& t, hipStream_t s) {
  switch (thin_width(t.N, CT)) {
    case 1: return launch_thin_t<1, TA, TB, CT>(t, s);
    case 2: return launch_thin_t<2, TA, TB, CT>(t, s);
    default: return launch_thin_t<4, TA, TB, CT>(t, s);
  }
}

template <bool CT>
hipError_t launch_thin(const Thin& t, bool ta, bool tb, hipStream_t s) {
  if (ta && tb) return launch_thin_op<true, true, CT>(t, s);
  if (ta) return launch_thin_op<true, false, CT>(t, s);
  if (tb) return launch_thin_op<false, true, CT>(t, s);
  return launch_thin_op<false, false, CT>(t, s);
}

Geometry thin_geometry(int64_t thin_rows, int64_t n, int K, bool few_cols) {
  const int v = thin_width(n, few_cols);
  const int64_t panels = ceil_div(thin_rows, 16);
  Geometry g;
  g.threads = 64 * kThinWaves;
  const int64_t per_panel = ceil_div(n, 16 * v);
  const int64_t cap = kMaxWorkItems / g.threads;
  g.tiles = per_panel * panels;
  g.workgroups = (per_panel < cap ? per_panel : cap) * panels;
  g.k_steps = ceil_div(K, 16 * kThinWaves);
  g.tile_m = few_cols ? 16 * v : 16;
  g.tile_n = few_cols ? 16 : 16 * v;
  return g;
}

// Smallest power of two that covers n (the kernels take 1, 2 or 4).
int padded_width(int n) {
  int w = 1;
  while (w < n) w *= 2;
  return w;
}

template <int RP, bool TA, bool TB>
hipError_t launch_rows_t(const Problem& p, hipStream_t s) {
  const int64_t nblocks = ceil_div(p.N, 16);
  const int64_t grid = nblocks < kMaxWorkItems / FewRows<RP>::THREADS
                           ? nblocks : kMaxWorkItems / FewRows<RP>::THREADS;
  hipLaunchKernelGGL((k_few_rows<RP, TA, TB>), dim3(static_cast<unsigned>(grid)),
                     dim3(FewRows<RP>::THREADS), 0, s, p, nblocks);
  return hipGetLastError();
}

template <int WP, bool TB>
hipError_t launch_cols_t(const Problem& p, hipStream_t s) {
  const int64_t nblocks = ceil_div(p.M, kRowsPerBlock);
  const int64_t grid = nblocks < kMaxWorkItems / kColThreads ? nblocks
                                                              : kMaxWorkItems / kColThreads;
  hipLaunchKernelGGL((k_few_cols<WP, TB>), dim3(static_cast<unsigned>(grid)), dim3(kColThreads), 0, s,
                     p, nblocks);
  return hipGetLastError();
}

}  // namespace

Geometry few_rows_geometry(int M, int N, int K) {
  if (!thin_on_valu(M, N)) return thin_geometry(M, N, K, false);
  const int rp = padded_width(M);
  return make_geometry(rp, N, K, rp, 16, FewRows<4>::KSWEEP, FewRows<4>::THREADS);
}

template <bool TA, bool TB>
hipError_t launch_rows_op(const Problem& p, hipStream_t s) {
  switch (padded_width(p.M)) {
    case 1: return launch_rows_t<1, TA, TB>(p, s);
    case 2: return launch_rows_t<2, TA, TB>(p, s);
    case 4: return launch_rows_t<4, TA, TB>(p, s);
    default: return hipErrorInvalidValue;  // more rows go to the matrix-core form
  }
}

hipError_t launch_few_rows(const Problem& p, hipStream_t s) {
  if (!thin_on_valu(p.M, p.N)) {
    const Thin t{p.M, p.N, p.K, p.alpha, p.beta, p.A, p.lda, p.B, p.ldb, p.C, p.ldc};
    return launch_thin<false>(t, p.trans_a, p.trans_b, s);
  }
  if (p.trans_a && p.trans_b) return launch_rows_op<true, true>(p, s);
  if (p.trans_a) return launch_rows_op<true, false>(p, s);
  if (p.trans_b) return launch_rows_op<false, true>(p, s);
  return launch_rows_op<false, false>(p, s);
}

Geometry few_cols_geometry(int M, int N, int K) {
  if (!thin_on_valu(N, M)) return thin_geometry(N, M, K, true);
  const int wp = padded_width(N);
  return make_geometry(M, wp, K, kRowsPerBlock, wp, FewCols<4>::KC, kColThreads);
}

template <bool TB>
hipError_t launch_cols_op(const Problem& p, hipStream_t s) {
  switch (padded_width(p.N)) {
    case 1: return launch_cols_t<1, TB>(p, s);
    case 2: return launch_cols_t<2, TB>(p, s);
    case 4: return launch_cols_t<4, TB>(p, s);
    default: return hipErrorInvalidValue;  // more columns go to the matrix-core form
  }
}

Geometry thin_panels_geometry(int M, int N, int K) { return thin_geometry(M, N, K, false); }

hipError_t launch_thin_panels(const Problem& p, hipStream_t s) {
  const Thin t{p.M, p.N, p.K, p.alpha, p.beta, p.A, p.lda, p.B, p.ldb, p.C, p.ldc};
  return launch_thin<false>(t, p.trans_a, p.trans_b, s);
}

hipError_t launch_few_cols(const Problem& p, hipStream_t s) {
  // C^T = B^T A^T: A' = B^T (row-major B is B^T stored transposed), B' = A^T
  // (row-major A is A^T stored transposed), C' = C^T stored transposed.
  // The vector-ALU form reads A by rows: not for a transposed A.
  if (p.trans_a || !thin_on_valu(p.N, p.M)) {
    const Thin t{p.N, p.M, p.K, p.alpha, p.beta, p.B, p.ldb, p.A, p.lda, p.C, p.ldc};
    return launch_thin<true>(t, !p.trans_b, !p.trans_a, s);
  }
  return p.trans_b ? launch_cols_op<true>(p, s) : launch_cols_op<false>(p, s);
}

}  // namespace sgemm
