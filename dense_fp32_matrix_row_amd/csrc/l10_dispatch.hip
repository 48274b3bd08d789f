// l10_dispatch.hip -- level 10: shape-aware dispatch over level 9's
// matrix-core tiles and the thin-problem kernels.
//
// A vendor BLAS is a collection of specialised kernels chosen at run time by
// problem size ([GEMM2], section on the size sweep against cuBLAS and why
// small matrices fall behind), where each hand-written rung of the pages has
// one fixed tiling.  This rung does the same with what the library has:
//   - M <= 16 or N <= 16: the thin kernels (a matrix-core tile would be
//     mostly empty rows or columns, and the problem is bound by reading the
//     other operand);
//   - a large problem whose M and N miss a multiple of the 256 x 128 (or
//     128 x 128) tile by at most 16: whole tiles over the largest multiple,
//     no per-element bounds logic (only the last K step masks when K is
//     ragged), plus the thin kernels on the fringe.  At 4097^3 this replaces
//     level 9's 2145 edge-checked 128 x 64 tiles by the 512 whole 256 x 128
//     tiles of 4096^3 (exactly two per CU) and two one-element-wide strips;
//   - anything else: level 9's own tile choice.
// Every output element is still computed by exactly one kernel; the regions
// are disjoint, so the launches need no ordering beyond the stream's.
#include "sgemm_internal.h"

namespace sgemm {
namespace {

enum class Plan { kFewRows, kFewCols, kTiles, kTilesWithFringe };

struct Decomp {
  Plan plan;
  Shape shape;  // matrix-core tile shape of the tile grid
  int Mm, Nm;   // extent of the tile grid
};

Decomp decompose(int M, int N) {
  if (M <= kThin) return {Plan::kFewRows, Shape::kSmall, 0, 0};
  if (N <= kThin) return {Plan::kFewCols, Shape::kSmall, 0, 0};
  for (Shape s : {Shape::kHuge, Shape::kLarge}) {
    const TileDims d = shape_dims(s);
    const int mr = M % d.bm, nr = N % d.bn;
    const int Mm = M - mr, Nm = N - nr;
    if (mr <= kThin && nr <= kThin && int64_t(Mm / d.bm) * (Nm / d.bn) >= d.min_tiles)
      return {mr == 0 && nr == 0 ? Plan::kTiles : Plan::kTilesWithFringe, s, Mm, Nm};
  }
  return {Plan::kTiles, pick_shape(M, N), M, N};
}

Geometry geometry10(int M, int N, int K) {
  const Decomp d = decompose(M, N);
  switch (d.plan) {
    case Plan::kFewRows: return few_rows_geometry(M, N, K);
    case Plan::kFewCols: return few_cols_geometry(M, N, K);
    default: return mfma_geometry(d.shape, d.Mm, d.Nm, K);
  }
}

hipError_t launch10(const Problem& p, hipStream_t s) {
  const Decomp d = decompose(p.M, p.N);
  switch (d.plan) {
    case Plan::kFewRows: return launch_few_rows(p, s);
    case Plan::kFewCols: return launch_few_cols(p, s);
    case Plan::kTiles: return launch_mfma(d.shape, p, s);
    case Plan::kTilesWithFringe: break;
  }
  Problem grid = p;
  grid.M = d.Mm;
  grid.N = d.Nm;
  hipError_t e = launch_mfma(d.shape, grid, s);
  if (e == hipSuccess && d.Nm < p.N) {
    // right fringe: rows [0, Mm), columns [Nm, N)
    Problem right = p;
    right.M = d.Mm;
    right.N = p.N - d.Nm;
    right.B = p.B + d.Nm;
    right.C = p.C + d.Nm;
    e = launch_few_cols(right, s);
  }
  if (e == hipSuccess && d.Mm < p.M) {
    // bottom fringe: rows [Mm, M), every column
    Problem bottom = p;
    bottom.M = p.M - d.Mm;
    bottom.A = p.A + d.Mm * p.lda;
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
