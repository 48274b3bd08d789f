// l10_dispatch.hip -- level 10: shape-aware dispatch over level 9's
// matrix-core tiles and the thin-problem kernels.
//
// A vendor BLAS is a collection of specialised kernels chosen at run time by
// problem size ([GEMM2], section on the size sweep against cuBLAS and why
// small matrices fall behind), where each hand-written rung of the pages has
// one fixed tiling.  This rung does the same with what the library has:
//   - M <= 16 or N <= 16: the thin kernels (a matrix-core tile would be
//     mostly empty rows or columns, and the problem is bound by reading the
//     other operand; l10_thin.hip gives them one 16-row MFMA block or
//     vector-ALU FMA chains);
//   - a large problem whose M and N miss a multiple of the 256 x 128 (or
//     128 x 128) tile by at most 16: whole tiles over the largest multiple,
//     no per-element bounds logic (only the last K step masks when K is
//     ragged), plus the thin kernels on the fringe.  Whole 256 x 128 and
//     128 x 128 tiles run l10_kloop.hip, the same tiles with their K loop
//     scheduled by hand.  At 4097^3 this replaces
//     level 9's 2145 edge-checked 128 x 64 tiles by the 512 whole 256 x 128
//     tiles of 4096^3 (exactly two per CU) and two one-element-wide strips;
//   - a deep K over a small tile grid: split K (l10_splitk.hip);
//   - anything else: the tile shape whose grid fills the CUs best, with two
//     K slices per stage where one block per CU would leave each SIMD a
//     single wavefront.
// Every output element is computed by exactly one tile or thin kernel (or,
// split, by one reduction over its slices); the regions are disjoint, so
// the launches need no ordering beyond the stream's.
#include "sgemm_internal.h"

namespace sgemm {
namespace {

enum class Plan { kFewRows, kFewCols, kTiles, kTilesWithFringe, kSplitK };

struct Decomp {
  Plan plan;
  Shape shape;      // matrix-core tile shape
  int Mm, Nm;       // extent of the tile grid (kTilesWithFringe)
  int64_t k_split;  // slice length (kSplitK)
};

constexpr int kCUs = 256;

// Fraction of the last round of blocks that is busy: tiles over whole
// rounds of one block per CU.
double round_fill(int64_t tiles) {
  const int64_t rounds = ceil_div(tiles, kCUs);
  return double(tiles) / double(rounds * kCUs);
}

// The rules below were fitted to sweeps of every tile shape and slice count
// on MI355X (dense_fp32_matrix_row_amd.autotune); the comments give the
// measurements that decided them.
Decomp decompose(int M, int N, int K) {
  if (M <= kThin) return {Plan::kFewRows, Shape::kSmall, M, N, K};
  if (N <= kThin) return {Plan::kFewCols, Shape::kSmall, M, N, K};

  // 1. At least two 256 x 128 tiles per CU (plus a fringe of <= 16): the
  //    big tile (4096^3: 138 TFLOP/s; 4097^3 with the fringe: 127).
  {
    const int mr = M % 256, nr = N % 128;
    const int64_t tiles = int64_t((M - mr) / 256) * ((N - nr) / 128);
    if (mr <= kThin && nr <= kThin && tiles >= 2 * kCUs)
      return {mr || nr ? Plan::kTilesWithFringe : Plan::kTiles, Shape::kHuge, M - mr, N - nr, K};
  }

  // 2. Deep K over less than one round of 128 x 128 tiles: split K so that
  //    about two work items per CU run (1024 x 1024 x 4096: 128 x 128 in
  //    8 slices 108 TFLOP/s against 38 unsplit; 1024 x 1024 x 8192: 127-128
  //    in 4-8 slices; 512 x 512 x 8192: 84-88 against 9).  Slices stay
  //    >= 256 deep (512 for the big tile) and at most 16.  (A full round,
  //    2048 x 2048 x 8192, runs unsplit: 148.5 against 144 in 2-4 slices.)
  const int64_t tiles128 = ceil_div(M, 128) * ceil_div(N, 128);
  if (K >= 2048 && K >= 2 * int64_t(M > N ? M : N) && tiles128 < kCUs) {
    Shape shape = Shape::kSmall;
    int64_t tiles = ceil_div(M, 64) * ceil_div(N, 64), min_slice = 256;
    if (M % 256 == 0 && N % 128 == 0 && int64_t(M / 256) * (N / 128) >= 64) {
      shape = Shape::kHuge;
      tiles = int64_t(M / 256) * (N / 128);
      min_slice = 512;
    } else if (tiles128 >= 16) {
      shape = Shape::kLarge;
      tiles = tiles128;
    }
    int64_t splits = ceil_div(2 * kCUs, tiles);
    if (splits > 16) splits = 16;
    if (splits > K / min_slice) splits = K / min_slice;
    if (splits >= 2) {
      const int64_t k_split = k_split_for(K, splits, shape_bk(shape));
      if (k_split < K) return {Plan::kSplitK, shape, M, N, k_split};
    }
  }

  // 3. 128 x 128 tiles (plus a fringe of <= 16) when they fill whole rounds
  //    of CUs: the assembly-loop tile (2048^3: 123-140 against 105-122 for
  //    any compiled tile; 2048 x 4096: 142-146).
  {
    const int mr = M % 128, nr = N % 128;
    const int64_t tiles = int64_t((M - mr) / 128) * ((N - nr) / 128);
    if (mr <= kThin && nr <= kThin && tiles >= kCUs && round_fill(tiles) >= 0.9) {
      return {mr || nr ? Plan::kTilesWithFringe : Plan::kTiles, Shape::kLarge, M - mr, N - nr, K};
    }
  }

  // 3b. A whole grid of >= 128 such tiles whose last round is partly idle:
  //     split K into s <= 4 slices, the s with the fewest rounds of work
  //     items per slice depth (ceil(tiles s / CUs) / s; ties to fewer
  //     slices): 3072^3 in 4 slices 135.6 against 119.7 for the 64 x 64
  //     tile (rule 4) and 113.6 unsplit; 1536^3 in 3 slices 91.0 against
  //     83.6 and 79.7.  (Below 128 tiles the 64 x 64 tile wins: 1024^3
  //     77.7 against at most 54 for split 128 x 128 tiles.)
  if (M % 128 == 0 && N % 128 == 0 && tiles128 >= 128 && K >= 1024) {
    int best = 1;
    double best_cost = double(ceil_div(tiles128, kCUs));
    for (int s = 2; s <= 4; ++s) {
      const double cost = double(ceil_div(tiles128 * s, kCUs)) / s;
      if (cost < best_cost - 1e-9) {
        best = s;
        best_cost = cost;
      }
    }
    if (best > 1) return {Plan::kSplitK, Shape::kLarge, M, N, k_split_for(K, best, 16)};
  }

  // 4. Everything else: 64 x 64 tiles with two K slices, up to three blocks
  //    per CU (1024^3: 66 against 56 unsliced; 3072^3: 115 against 73 for
  //    128 x 128 tiles, whose 576 tiles leave the third round 1/4 full;
  //    it beats the 128 x 64 tile at every size measured, 512^3 to 4096^3).
  return {Plan::kTiles, Shape::kSmallSliced, M, N, K};
}

Geometry geometry10(int M, int N, int K) {
  const Decomp d = decompose(M, N, K);
  switch (d.plan) {
    case Plan::kFewRows: return few_rows_geometry(M, N, K);
    case Plan::kFewCols: return few_cols_geometry(M, N, K);
    case Plan::kSplitK: return tiles_split_geometry(d.shape, M, N, K, d.k_split);
    default: return tiles_geometry(d.shape, d.Mm, d.Nm, K);
  }
}

hipError_t launch10(const Problem& p, hipStream_t s) {
  const Decomp d = decompose(p.M, p.N, p.K);
  switch (d.plan) {
    case Plan::kFewRows: return launch_few_rows(p, s);
    case Plan::kFewCols: return launch_few_cols(p, s);
    case Plan::kTiles: return launch_tiles(d.shape, p, s);
    case Plan::kSplitK: return launch_splitk(d.shape, d.k_split, p, s);
    case Plan::kTilesWithFringe: break;
  }
  Problem grid = p;
  grid.M = d.Mm;
  grid.N = d.Nm;
  hipError_t e = launch_tiles(d.shape, grid, s);
  if (e == hipSuccess && d.Nm < p.N) {
    // right fringe: rows [0, Mm), columns [Nm, N) (B's columns are its rows
    // when it is stored transposed)
    Problem right = p;
    right.M = d.Mm;
    right.N = p.N - d.Nm;
    right.B = p.B + (p.trans_b ? d.Nm * p.ldb : d.Nm);
    right.C = p.C + d.Nm;
    e = launch_few_cols(right, s);
  }
  if (e == hipSuccess && d.Mm < p.M) {
    // bottom fringe: rows [Mm, M), every column
    Problem bottom = p;
    bottom.M = p.M - d.Mm;
    bottom.A = p.A + (p.trans_a ? d.Mm : d.Mm * p.lda);
    bottom.C = p.C + d.Mm * p.ldc;
    e = launch_few_rows(bottom, s);
  }
  return e;
}

}  // namespace

const LevelDesc* level10() {
  static const LevelDesc d = {"L10_shape_dispatch", geometry10, launch10};
  return &d;
}

}  // namespace sgemm
