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
//   - a deep K over 64-255 tiles of 64 x 64, or K >= 2048 over a wide,
//     shallow grid of 64-128 of them: split K (l10_splitk.hip);
//   - otherwise one of the three assembly-loop tiles of l10_kloop.hip
//     (256 x 128, 128 x 128, 64 x 64), the one that leaves the busiest CU
//     the least work, with partial edge tiles, or with whole tiles and a
//     fringe: one row and / or one column (4097^3: the 512 whole tiles of
//     4096^3 and two one-element strips; 1025^3: 256 tiles of 64 x 64) is
//     summed by the tiles' own blocks from the operands they hold in LDS,
//     in the same launch; up to 16 beside the two large tiles by the thin
//     kernels;
//   - small problems (fewer than 128 tiles of 64 x 64): the thin
//     matrix-core kernel over 16-row panels of C.
// Every output element is computed by exactly one tile or thin kernel (or,
// split, by one reduction over its slices); the regions are disjoint, so
// the launches need no ordering beyond the stream's.
#include "sgemm.h"
#include "sgemm_internal.h"

namespace sgemm {
namespace {

enum class Plan { kFewRows, kFewCols, kTiles, kTilesWithFringe, kSplitK, kThinPanels };

struct Decomp {
  Plan plan;
  Shape shape;      // matrix-core tile shape
  int Mm, Nm;       // extent of the tile grid (kTilesWithFringe)
  int64_t k_split;  // slice length (kSplitK)
};

constexpr int kCUs = 256;

// The rules below were fitted to sweeps of every tile shape and slice count
// on MI355X (dense_fp32_matrix_row_amd.autotune); the comments give the
// measurements that decided them.  The sweep's table of record is checked
// by tests/test_autotune_cpu.py: every swept shape must still get the plan
// and tile configuration recorded for it, and that configuration must be
// within the sweep's tolerance of the fastest one measured.
// A packed problem of this shape (lda = K, ldb = N, row-major), for the
// decisions made from M, N and K alone.
Problem packed(int M, int N, int K) {
  Problem p{};
  p.M = M;
  p.N = N;
  p.K = K;
  p.lda = K;
  p.ldb = N;
  p.ldc = N;
  return p;
}

Decomp decompose(int M, int N, int K) {
  if (M <= kThin) return {Plan::kFewRows, Shape::kSmall, M, N, K};
  if (N <= kThin) return {Plan::kFewCols, Shape::kSmall, M, N, K};

  const int64_t tiles64 = ceil_div(M, 64) * ceil_div(N, 64);
  const bool deep = K >= 2048 && K >= 2 * int64_t(M > N ? M : N);

  // 1. A deep K over less than one round of 64 x 64 tiles (but >= 64 of
  //    them): the 64 x 64 assembly loop split into the most K parts (<= 16,
  //    each >= 256 deep) that keep at most two work items per CU
  //    (l10_splitk.hip: workspace planes from the library's pool, an
  //    in-order reduction applying alpha and beta): 512 x 512 x 8192 (64
  //    tiles) in 8 parts 85.8 TFLOP/s (in 4: 87.0); 768 x 768 x 4096 (144
  //    tiles) in 3: 82.7 against 70.2 on compiled tiles.
  if (deep && tiles64 >= 64 && tiles64 < kCUs) {
    int64_t parts = 2 * kCUs / tiles64;
    if (parts > 16) parts = 16;
    if (parts > K / 256) parts = K / 256;
    if (parts >= 2) {
      const int64_t k_split = k_split_for(K, parts, shape_bk(Shape::kSmallDeep));
      if (k_split < K) return {Plan::kSplitK, Shape::kSmallDeep, M, N, k_split};
    }
  }

  // 1b. A wide, shallow grid of 64-128 tiles of 64 x 64 (one side 48-128
  //    rows or columns, the other thousands) with K >= 2048, which rule 1
  //    leaves alone because K is not twice the long side: split into the
  //    parts that make one round of work items, 4 over <= 64 tiles and 2
  //    over <= 128 (more parts measured slower: items of at most ~1000 k
  //    pay their per-launch start more often).  Sweeps against the plans
  //    without it: 64 x 4096 x 4096 65.1 TFLOP/s against 39.4 on the thin
  //    panels, 4096 x 64 x 4096 64.9 / 39.4, 64 x 4096 x 2048 42.8 / 37.4,
  //    128 x 4096 x 4096 90.1 / 65.5 on unsplit 64 x 64 tiles, 64 x 8192 x
  //    8192 104.7 / 69.0, 96 x 4096 x 4096 67.2 / 48.6, 48 x 8192 x 4096
  //    65.7 / 48.3, 256 x 2048 x 2048 66.5 / 59.3.  Thinner sides stay on
  //    the thin panels (32 x 4096 x 4096: 34.1 there, 32.1 split), and so
  //    do shallower K (64 x 4096 x 1024: 32.5 there, at most 25.0 split).
  const int64_t short_side = M < N ? M : N;
  if (!deep && K >= 2048 && short_side >= 48 && tiles64 >= 64 && tiles64 <= 128) {
    const int64_t parts = tiles64 <= 64 ? 4 : 2;
    const int64_t k_split = k_split_for(K, parts, shape_bk(Shape::kSmallDeep));
    if (k_split < K) return {Plan::kSplitK, Shape::kSmallDeep, M, N, k_split};
  }

  // 2. A grid of >= 128 tiles of 64 x 64: whichever of the three
  //    assembly-loop tiles leaves the busiest CU the least work,
  //    ceil(tiles / CUs) x tile area / efficiency, the efficiency measured
  //    for that tile at that many tiles per CU (256 x 128: 0.955 from two
  //    per CU, 0.85 with one; 128 x 128: 0.935 / 0.895; 64 x 64, 64-deep
  //    stages over four K-slice wavefronts: 0.89).  A tile counts whole
  //    tiles only where M and N miss a multiple by one (the tiles' own
  //    blocks sum that row and column, where the grid has enough tiles for
  //    their shares: 4097^3 on 512 tiles of 256 x 128 and two one-element
  //    strips, 148 against 121 for the vendor BLAS), or, for the 256 x 128
  //    and 128 x 128 tiles, by at most 16 (the rest goes to the thin
  //    kernels), and partial edge tiles otherwise.  Picks on the
  //    sweeps: 256 x 128 at 4096^3 (150-152), 4000^3 (145 against 137 for
  //    64 x 64), 5000 x 3000 x 2000 (133.5); 128 x 128 at 2048^3 (140-141
  //    against 132.6), 1792^3 (109 against 100), 2048 x 4096, 1024 x 4096 x
  //    1024 (130 against 119), 2048 x 2048 x 8192 (148), 6000^3 (145.4);
  //    64 x 64 at 1024^3 (89-93 against <= 80 for compiled tiles), 1536^3
  //    (94.7), 2500^3 (114.8), 3000^3 (132.8; compiled: 101.6), 3072^3
  //    (140.6), 3584^3 (135.3), 4608^3 (140.2 against 128.5 for 648 tiles
  //    of 256 x 128), 5120^3 (146.2 against 119.2 for 800), 1024 x 1024 x
  //    4096 / 8192 (123 / 130.5).
  if (tiles64 >= 128) {
    struct Candidate {
      Shape shape;
      int bm, bn;
      double eff_one, eff_more;  // efficiency with one / several tiles per CU
    };
    static const Candidate candidates[] = {{Shape::kHuge, 256, 128, 0.85, 0.955},
                                           {Shape::kLarge, 128, 128, 0.895, 0.935},
                                           {Shape::kSmallDeep, 64, 64, 0.89, 0.89}};
    Decomp best{Plan::kTiles, Shape::kSmallDeep, M, N, K};
    double best_cost = 0.0;
    for (const Candidate& c : candidates) {
      const int mr = M % c.bm, nr = N % c.bn;
      // one row and / or column that the tiles' blocks sum (enough tiles
      // for their shares), or up to 16 beside the large tiles for the thin
      // kernels.  The 64 x 64 tile's alternative is a grid with partial
      // edge tiles: its fringe variant only where that leaves the busiest
      // CU fewer tiles (1025^3: 256 tiles against 289, 40.5 -> 28.0 us; at
      // the same count, 1537^3: 576 against 625, the edges measured 79 us
      // against 88)
      bool fused = mr <= 1 && nr <= 1 && (mr || nr) &&
                   tiles_fringe_fits(c.shape, packed(M, N, K), M - mr, N - nr);
      if (fused && c.shape == Shape::kSmallDeep)
        fused = ceil_div(int64_t(M / c.bm) * (N / c.bn), kCUs) <
                ceil_div(ceil_div(M, c.bm) * ceil_div(N, c.bn), kCUs);
      const bool fringe = fused || (c.shape != Shape::kSmallDeep && mr <= kThin && nr <= kThin &&
                                    M - mr > 0 && N - nr > 0);
      const int Mm = fringe ? M - mr : M, Nm = fringe ? N - nr : N;
      const int64_t per_cu = ceil_div(ceil_div(Mm, c.bm) * ceil_div(Nm, c.bn), kCUs);
      const double cost = double(per_cu) * c.bm * c.bn / (per_cu > 1 ? c.eff_more : c.eff_one);
      if (best_cost == 0.0 || cost < best_cost) {
        const Plan plan = fringe && (mr || nr) ? Plan::kTilesWithFringe : Plan::kTiles;
        best = {plan, c.shape, Mm, Nm, K};
        best_cost = cost;
      }
    }
    return best;
  }

  // 3. Everything else (fewer than 128 tiles of 64 x 64, and for a deep K
  //    fewer than 64): the thin
  //    matrix-core kernel over 16-row panels of C, its columns in blocks of
  //    16 (64 when there are many), K over sixteen wavefronts per block, so
  //    that the grid has panels x column blocks workgroups instead of a few
  //    dozen tiles.  Against compiled 64 x 64 tiles (and, for deep K, their
  //    split): 256^3 10.4 -> 6.1 us, 400^3 17.2 -> 8.4, 200 x 300 x 2000
  //    57.8 -> 10.8, 128 x 512 x 4096 24.7 -> 16.7, 300 x 300 x 3000
  //    31.5 -> 23.2; 256 x 256 x 8192 and 200 x 200 x 16384 the same.
  //    Against 64 x 64 loop tiles at 64-127 of them: 512^3 14.3 -> 11.3 us,
  //    600^3 17.3 -> 15.6, 512 x 512 x 1536 28.8 -> 21.5 (at 144 and more,
  //    768^3 and 900^3, the loop tiles are faster).
  return {Plan::kThinPanels, Shape::kSmallSliced, M, N, K};
}

// A fringe of at most one row and one column runs in the tiles' launch
// (l10_kloop.hip's fringe variant) where its offsets fit; the plan query
// assumes packed operands (lda = K, ldb = N for row-major storage), the
// launch checks the caller's and falls back to the grid plus the thin
// kernels.
bool one_launch_fringe(const Decomp& d, const Problem& p) {
  return d.plan == Plan::kTilesWithFringe && tiles_fringe_fits(d.shape, p, d.Mm, d.Nm);
}

bool one_launch_fringe(const Decomp& d, int M, int N, int K) { return one_launch_fringe(d, packed(M, N, K)); }

Geometry geometry10(int M, int N, int K) {
  const Decomp d = decompose(M, N, K);
  switch (d.plan) {
    case Plan::kFewRows: return few_rows_geometry(M, N, K);
    case Plan::kFewCols: return few_cols_geometry(M, N, K);
    case Plan::kSplitK: return tiles_split_geometry(d.shape, M, N, K, d.k_split);
    case Plan::kThinPanels: return thin_panels_geometry(M, N, K);
    default: return tiles_geometry(d.shape, d.Mm, d.Nm, K);
  }
}

}  // namespace

PlanInfo plan10(int M, int N, int K) {
  PlanInfo info{SGEMM_PLAN_NONE, 0, 0};
  if (M <= 0 || N <= 0) return info;
  if (K <= 0) return {SGEMM_PLAN_SCALE, 1, 0};
  const Decomp d = decompose(M, N, K);
  switch (d.plan) {
    case Plan::kFewRows: return {SGEMM_PLAN_FEW_ROWS, 1, 0};
    case Plan::kFewCols: return {SGEMM_PLAN_FEW_COLS, 1, 0};
    case Plan::kTiles: return {SGEMM_PLAN_TILES, 1, 0};
    case Plan::kThinPanels: return {SGEMM_PLAN_THIN_PANELS, 1, 0};
    case Plan::kSplitK:
      return {SGEMM_PLAN_SPLIT_K, 2,
              ceil_div(K, d.k_split) * int64_t(M) * int64_t(N) * int64_t(sizeof(float))};
    case Plan::kTilesWithFringe:
      return {SGEMM_PLAN_TILES_FRINGE, one_launch_fringe(d, M, N, K) ? 1 : 1 + (d.Nm < N) + (d.Mm < M), 0};
  }
  return info;
}

hipError_t launch10_with(const Problem& p, hipStream_t s, Workspace w) {
  const Decomp d = decompose(p.M, p.N, p.K);
  switch (d.plan) {
    case Plan::kFewRows: return launch_few_rows(p, s);
    case Plan::kFewCols: return launch_few_cols(p, s);
    case Plan::kTiles: return launch_tiles(d.shape, p, s);
    case Plan::kSplitK: return launch_splitk(d.shape, d.k_split, p, s, w);
    case Plan::kThinPanels: return launch_thin_panels(p, s);
    case Plan::kTilesWithFringe: break;
  }
  if (one_launch_fringe(d, p)) return launch_tiles_fringe(d.shape, p, d.Mm, d.Nm, s);
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

namespace {

hipError_t launch10(const Problem& p, hipStream_t s) { return launch10_with(p, s, Workspace::kPool); }

}  // namespace

const LevelDesc* level10() {
  static const LevelDesc d = {"L10_shape_dispatch", geometry10, launch10};
  return &d;
}

}  // namespace sgemm
