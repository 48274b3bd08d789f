// l9_mfma.hip -- level 9: the level-8 pipeline with the FMA core moved onto
// the FP32 matrix cores (v_mfma_f32_32x32x2_f32 and v_mfma_f32_16x16x4_f32:
// 32 x 32 x 2 and 16 x 16 x 4 products, full float32 inputs and
// accumulators, 2048 / 1024 FMAs per instruction per wavefront).
//
// None of the pages programs matrix instructions for FP32 ([L04] section 5.5
// only names them as what libraries add on top of tiling); GEMM is a dense
// contraction, so on gfx950 the FMA core belongs on the matrix cores.  The
// pages' xf32 reduced-precision modes are not used (gfx950 has none for FP32,
// and ~10-bit inputs would miss the 1e-5 normalised error bound).
//
// The kernel template and its tile shapes are in l9_tile.h; this file holds
// level 9's shape choice and the per-shape entry points (untransposed
// operands here, the transposed orientations in l9_mfma_ops.hip).
//
// The staging (A transposed into LDS, 128-bit global loads, element-wise
// loads only for partial groups at the K/N edges, zero-fill beyond M/N/K),
// the double-buffered one-barrier pipeline and the XCD-aware grouped block
// order are those of level 8.  The summation order inside an instruction is the
// hardware's, so results differ from levels 0-8 in the last bits (all within
// the float32 rounding bound); integer-valued inputs still give exact results.
#include "l9_tile.h"

namespace sgemm {

Shape pick_shape(int M, int N) {
  const int64_t tiles128 = ceil_div(M, 128) * ceil_div(N, 128);
  if (M % TileHuge::BM == 0 && N % TileHuge::BN == 0 &&
      (int64_t(M) / TileHuge::BM) * (N / TileHuge::BN) >= 2 * kCUs)
    return Shape::kHuge;
  if (M % TileLarge::BM == 0 && N % TileLarge::BN == 0 && tiles128 >= kCUs)
    return Shape::kLarge;
  if (int64_t(M) * N >= int64_t(2048) * 2048) return Shape::kMid;
  return Shape::kSmall;
}

TileDims shape_dims(Shape shape) {
  switch (shape) {
    case Shape::kHuge: return {TileHuge::BM, TileHuge::BN, 2 * kCUs};
    case Shape::kLarge: return {TileLarge::BM, TileLarge::BN, kCUs};
    case Shape::kMid: return {TileMid::BM, TileMid::BN, 0};
    case Shape::kLargeSliced: return {TileLargeSliced::BM, TileLargeSliced::BN, 0};
    case Shape::kSmallSliced: return {TileSmallSliced::BM, TileSmallSliced::BN, 0};
    default: return {TileSmall::BM, TileSmall::BN, 0};
  }
}

Geometry mfma_geometry(Shape shape, int M, int N, int K) {
  switch (shape) {
    case Shape::kHuge: return tile_geometry<TileHuge>(M, N, K);
    case Shape::kLarge: return tile_geometry<TileLarge>(M, N, K);
    case Shape::kMid: return tile_geometry<TileMid>(M, N, K);
    case Shape::kLargeSliced: return tile_geometry<TileLargeSliced>(M, N, K);
    case Shape::kSmallSliced: return tile_geometry<TileSmallSliced>(M, N, K);
    default: return tile_geometry<TileSmall>(M, N, K);
  }
}

hipError_t launch_mfma(Shape shape, const Problem& p, hipStream_t s) {
  if (p.trans_a && p.trans_b) return launch_mfma_tt(shape, p, s);
  if (p.trans_a) return launch_mfma_tn(shape, p, s);
  if (p.trans_b) return launch_mfma_nt(shape, p, s);
  return launch_shape_t<false, false>(shape, p, s);
}

int shape_bk(Shape shape) {
  switch (shape) {
    case Shape::kHuge: return TileHuge::BK;
    case Shape::kLarge: return TileLarge::BK;
    case Shape::kMid: return TileMid::BK;
    case Shape::kLargeSliced: return TileLargeSliced::BK;
    case Shape::kSmallSliced: return TileSmallSliced::BK;
    // level 10's 64 x 64 loop tile: 64-deep stages (also a multiple of the
    // BK of the compiled tile that stands in for it)
    case Shape::kSmallDeep: return 64;
    default: return TileSmall::BK;
  }
}

Geometry mfma_split_geometry(Shape shape, int M, int N, int K, int64_t k_split) {
  switch (shape) {
    case Shape::kHuge: return split_geometry<TileHuge>(M, N, K, k_split);
    case Shape::kLarge: return split_geometry<TileLargeSplit>(M, N, K, k_split);
    case Shape::kMid: return split_geometry<TileMid>(M, N, K, k_split);
    case Shape::kLargeSliced: return split_geometry<TileLargeSliced>(M, N, K, k_split);
    case Shape::kSmallSliced: return split_geometry<TileSmallSliced>(M, N, K, k_split);
    default: return split_geometry<TileSmall>(M, N, K, k_split);
  }
}

hipError_t launch_mfma_split(Shape shape, const Problem& p, int64_t k_split, float* ws,
                             hipStream_t s) {
  if (p.trans_a && p.trans_b) return launch_mfma_split_tt(shape, p, k_split, ws, s);
  if (p.trans_a) return launch_mfma_split_tn(shape, p, k_split, ws, s);
  if (p.trans_b) return launch_mfma_split_nt(shape, p, k_split, ws, s);
  return launch_split_shape_t<false, false>(shape, p, k_split, ws, s);
}

namespace {

Geometry geometry9(int M, int N, int K) { return mfma_geometry(pick_shape(M, N), M, N, K); }

hipError_t launch9(const Problem& p, hipStream_t s) { return launch_mfma(pick_shape(p.M, p.N), p, s); }

}  // namespace

const LevelDesc* level9() {
  static const LevelDesc d = {"L9_mfma_f32", geometry9, launch9};
  return &d;
}

}  // namespace sgemm
