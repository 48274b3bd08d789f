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
//   - the tile shape whose grid fills the CUs best: 128 x 128 tiles, or the
//     64 x 64 tile whose 64-deep stages are split over four wavefronts
//     (l10_kloop.hip);
//   - a deep K over a small tile grid: split K (l10_splitk.hip);
//   - anything else: compiled 64 x 64 tiles with two K slices per stage.
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
  //    big tile (4096^3: 150-152 TFLOP/s; 4097^3 with the fringe: 143).
  {
    const int mr = M % 256, nr = N % 128;
    const int64_t tiles = int64_t((M - mr) / 256) * ((N - nr) / 128);
    if (mr <= kThin && nr <= kThin && tiles >= 2 * kCUs)
      return {mr || nr ? Plan::kTilesWithFringe : Plan::kTiles, Shape::kHuge, M - mr, N - nr, K};
  }

  // 2. 128 x 128 tiles (plus a fringe of <= 16) that fill whole rounds of
  //    CUs, or one round at least 70 % full (2048^3: 140.8 against 132.6
  //    for the 64 x 64 tile below; 1792^3, 196 tiles: 108.5 against 100.7;
  //    2048 x 4096: 147; 1024 x 4096 x 1024: 130 against 119).
  {
    const int mr = M % 128, nr = N % 128;
    const int64_t tiles = int64_t((M - mr) / 128) * ((N - nr) / 128);
    const bool fills = tiles >= kCUs ? round_fill(tiles) >= 0.9 : tiles * 10 >= kCUs * 7;
    if (mr <= kThin && nr <= kThin && fills)
      return {mr || nr ? Plan::kTilesWithFringe : Plan::kTiles, Shape::kLarge, M - mr, N - nr, K};
  }

  // 3. A whole grid of >= 64 tiles of 64 x 64: the deep-stage 64 x 64
  //    loop (four K-slice wavefronts per tile; two blocks fit a CU), which
  //    balances over the CUs where bigger tiles leave a round partly idle
  //    (1024^3: 89.3 against 76.5 for the best compiled tile; 1280^3: 91.5;
  //    1536^3: 94.7; 3072^3: 140.6 against 135.2 for 128 x 128 tiles in 4
  //    K parts; 3584^3: 135.3; 1024 x 2048 x 4096: 133.8; 1024 x 1024 x
  //    8192: 130.5 against 128 for split 128 x 128 tiles).  A deep K over
  //    less than one round of these tiles is split into the most parts
  //    (<= 16, each >= 256 deep) that keep at most two work items per CU:
  //    512 x 512 x 8192 (64 tiles) in 8 parts 85.8 (in 4: 87.0);
  //    768 x 768 x 4096 (144 tiles) in 3: 82.7 against 70.2 before.
  const int64_t tiles64 = ceil_div(M, 64) * ceil_div(N, 64);
  if (M % 64 == 0 && N % 64 == 0 && tiles64 >= 64) {
    if (K >= 2048 && K >= 2 * int64_t(M > N ? M : N) && tiles64 < kCUs) {
      int64_t parts = 2 * kCUs / tiles64;
      if (parts > 16) parts = 16;
      if (parts > K / 256) parts = K / 256;
      if (parts >= 2) {
        const int64_t k_split = k_split_for(K, parts, shape_bk(Shape::kSmallDeep));
        if (k_split < K) return {Plan::kSplitK, Shape::kSmallDeep, M, N, k_split};
      }
    }
    return {Plan::kTiles, Shape::kSmallDeep, M, N, K};
  }

  // 4. Deep K over less than one round of 128 x 128 tiles, M or N not a
  //    multiple of 64: split K on compiled tiles so that about two work
  //    items per CU run (slices >= 256 deep (512 for the big tile), <= 16).
  const int64_t tiles128 = ceil_div(M, 128) * ceil_div(N, 128);
  if (K >= 2048 && K >= 2 * int64_t(M > N ? M : N) && tiles128 < kCUs) {
    Shape shape = Shape::kSmall;
    int64_t tiles = tiles64, min_slice = 256;
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

  // 5. Everything else: compiled 64 x 64 tiles with two K slices, up to
  //    three blocks per CU (3000^3: 101.5; 256^3: 3.2; it beats the
  //    128 x 64 tile at every size measured, 512^3 to 4096^3).
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
