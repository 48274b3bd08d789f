// sgemm_internal.h -- types and device helpers shared by the kernels of
// libsgemm (not installed; the public interface is include/sgemm.h).
//
// Citation keys ([SIX], [CP04], [L04], [GEMM2]) are defined in sgemm.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sgemm {

// One call's arguments, with the leading dimensions widened to 64 bits so
// that row*ld never overflows (the page kernels index with int products,
// which wrap past 46340^2 elements).
struct Problem {
  int M, N, K;
  float alpha, beta;
  const float* A;
  int64_t lda;
  const float* B;
  int64_t ldb;
  float* C;
  int64_t ldc;
  // op(A) = A^T: A is stored K x M (row stride lda >= M); op(B) = B^T: B is
  // stored N x K (ldb >= K).  Only the dispatching rung and the kernels it
  // composes read these; levels 0-9 are reached with both false.
  bool trans_a = false, trans_b = false;
};

// Launch geometry of one level for one shape.
struct Geometry {
  int64_t workgroups;  // blocks launched (tiles are walked grid-stride when
                       // there are more tiles than blocks)
  int threads;         // threads per block
  int64_t k_steps;     // K phases per tile: ceil(K / BK)
  int tile_m, tile_n;  // C tile per block
  int64_t tiles;       // tiles of C
};

using GeometryFn = Geometry (*)(int M, int N, int K);
using LaunchFn = hipError_t (*)(const Problem&, hipStream_t);

struct LevelDesc {
  const char* name;
  GeometryFn geometry;
  LaunchFn launch;
};

// Blocks per launch are capped so that blocks * threads stays below 2^31
// work-items (the dispatch packet's grid size is 32-bit); tiles beyond the
// cap are walked grid-stride by the same blocks.
constexpr int64_t kMaxWorkItems = int64_t(1) << 31;

__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) {
  return (a + b - 1) / b;
}

inline Geometry make_geometry(int M, int N, int K, int tile_m, int tile_n,
                              int bk, int threads) {
  Geometry g;
  g.tile_m = tile_m;
  g.tile_n = tile_n;
  g.threads = threads;
  g.tiles = ceil_div(M, tile_m) * ceil_div(N, tile_n);
  const int64_t cap = kMaxWorkItems / threads;
  g.workgroups = g.tiles < cap ? g.tiles : cap;
  g.k_steps = ceil_div(K, bk);
  return g;
}

// MI355X dispatches consecutive workgroup ids round-robin to its 8 XCDs,
// each with its own L2.  This maps block `bid` of `nblocks` to a logical id
// such that XCD x (= bid % 8) gets the x-th contiguous range of ids, so that
// neighbouring tiles (which share operand panels) share one L2.
__device__ __forceinline__ int64_t xcd_contiguous(int64_t bid, int64_t nblocks) {
  const int64_t q = nblocks / 8, r = nblocks % 8;
  const int64_t x = bid % 8, local = bid / 8;
  return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + local;
}

// The epilogue of every level: alpha*acc + beta*c, with C read only when
// beta != 0 (BLAS convention; the page kernels read C unconditionally).
__device__ __forceinline__ float epilogue(float acc, float alpha, float beta,
                                          const float* c) {
  const float r = alpha * acc;
  return beta == 0.0f ? r : fmaf(beta, *c, r);
}

// 128-bit global accesses need only 4-byte alignment on gfx950 (the compiler
// itself emits global_load_dwordx4 / global_store_dwordx4 for 16-byte copies
// of float data), so the vector paths below run for any row stride and any
// float-aligned base; the "alignment promise" of a float4 cast that [GEMM2]
// kernel 6 relies on is not needed for global memory here.
__device__ __forceinline__ float4 ld_global4(const float* p) {
  float4 v;
  __builtin_memcpy(&v, p, sizeof(v));
  return v;
}
__device__ __forceinline__ void st_global4(float* p, float4 v) {
  __builtin_memcpy(p, &v, sizeof(v));
}

// Four consecutive elements [col, col+4) of one row, zero outside
// [0, ncols) or when the row is out of range (the zero-fill boundary rule of
// [L04] section 2.5).  A full group is one 128-bit load; a partial group at
// the edge falls back to element loads (never the whole-group drop of [SIX]
// K6).
__device__ __forceinline__ float4 load4(const float* __restrict__ row_ptr,
                                        int64_t col, int64_t ncols,
                                        bool row_ok) {
  float4 v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  if (!row_ok) return v;
  if (col + 3 < ncols) {
    v = ld_global4(row_ptr + col);
  } else {
    if (col + 0 < ncols) v.x = row_ptr[col + 0];
    if (col + 1 < ncols) v.y = row_ptr[col + 1];
    if (col + 2 < ncols) v.z = row_ptr[col + 2];
    if (col + 3 < ncols) v.w = row_ptr[col + 3];
  }
  return v;
}

// Epilogue for four consecutive outputs C[row][col .. col+3] (only those
// below N are written; c points at C[row][col]).
__device__ __forceinline__ void store4(float* __restrict__ c, int64_t col,
                                       int64_t N, float4 acc, float alpha,
                                       float beta) {
  if (col + 3 < N) {
    float4 r = make_float4(alpha * acc.x, alpha * acc.y, alpha * acc.z,
                           alpha * acc.w);
    if (beta != 0.0f) {
      const float4 old = ld_global4(c);
      r.x = fmaf(beta, old.x, r.x);
      r.y = fmaf(beta, old.y, r.y);
      r.z = fmaf(beta, old.z, r.z);
      r.w = fmaf(beta, old.w, r.w);
    }
    st_global4(c, r);
  } else {
    if (col + 0 < N) c[0] = epilogue(acc.x, alpha, beta, c + 0);
    if (col + 1 < N) c[1] = epilogue(acc.y, alpha, beta, c + 1);
    if (col + 2 < N) c[2] = epilogue(acc.z, alpha, beta, c + 2);
    if (col + 3 < N) c[3] = epilogue(acc.w, alpha, beta, c + 3);
  }
}

// C <- beta*C over the M x N window (the K == 0 / alpha == 0 quick return).
hipError_t launch_scale(const Problem& p, hipStream_t stream);

// Level 9's matrix-core tile shapes, which the dispatching rung composes:
// Huge 256 x 128, Large 128 x 128, Mid 128 x 64, Small 64 x 64 block tiles,
// and 128 x 128 / 64 x 64 tiles whose stages are cut into two K slices
// (twice the wavefronts per tile; their sums meet in LDS).  SmallDeep is
// level 10's 64 x 64 assembly-loop tile (64-deep stages over four K-slice
// wavefronts); where that kernel does not fit, SmallSliced stands in.
enum class Shape { kHuge, kLarge, kMid, kSmall, kLargeSliced, kSmallSliced, kSmallDeep };
struct TileDims {
  int bm, bn;         // block tile
  int64_t min_tiles;  // tiles a problem needs before level 9 picks the shape
};
Shape pick_shape(int M, int N);  // level 9's own choice for a problem
TileDims shape_dims(Shape shape);
Geometry mfma_geometry(Shape shape, int M, int N, int K);
hipError_t launch_mfma(Shape shape, const Problem& p, hipStream_t s);
// Level 10's whole-tile kernels with their K loop in assembly
// (l10_kloop.hip), for the Huge (256 x 128), Large (128 x 128) and
// SmallDeep (64 x 64) shapes, any operand orientation, any M and N (edge
// tiles load and store only inside the matrix): buffer offsets below
// 2^31.  launch_tiles runs one where it fits, else the compiled tile
// kernel.
bool kloop_fits(Shape shape, const Problem& p);
hipError_t launch_tiles(Shape shape, const Problem& p, hipStream_t s);
Geometry tiles_geometry(Shape shape, int M, int N, int K);  // of launch_tiles, dense row-major
// A loop tile's fringe variant, one launch: whole tiles over the first
// Mm x Nm of C (multiples of the tile) and, summed by the same blocks, row
// M - 1 when p.M == Mm + 1 and column N - 1 when p.N == Nm + 1.  Fits when
// the grid has enough tiles for each block's share of the fringe (256 x
// 128: 4 x 8 tiles, 128 x 128: 8 x 8, 64 x 64: 16 x 16) and the buffer
// offsets (down to row M - 1 and across to column N - 1) stay below 2^31;
// launch_tiles_fringe returns hipErrorInvalidValue, enqueueing nothing,
// where it does not.
bool tiles_fringe_fits(Shape shape, const Problem& p, int Mm, int Nm);
hipError_t launch_tiles_fringe(Shape shape, const Problem& p, int Mm, int Nm, hipStream_t s);
// The same kernels over K slices (see launch_mfma_split): work item (tile,
// slice) stores raw sums into plane `slice` of ws.
hipError_t launch_tiles_split(Shape shape, const Problem& p, int64_t k_split, float* ws,
                              hipStream_t s);
Geometry tiles_split_geometry(Shape shape, int M, int N, int K, int64_t k_split);
// Split K over the same tiles: the K range is cut into slices of k_split
// (a multiple of the shape's BK) and each (tile, slice) is one work item
// that stores raw float32 sums into its slice's M x N plane of ws.
int shape_bk(Shape shape);
Geometry mfma_split_geometry(Shape shape, int M, int N, int K, int64_t k_split);
hipError_t launch_mfma_split(Shape shape, const Problem& p, int64_t k_split, float* ws,
                             hipStream_t s);
// The transposed orientations (l9_mfma_{tn,nt,tt}.hip): tn = A transposed,
// nt = B transposed, tt = both.
hipError_t launch_mfma_tn(Shape shape, const Problem& p, hipStream_t s);
hipError_t launch_mfma_nt(Shape shape, const Problem& p, hipStream_t s);
hipError_t launch_mfma_tt(Shape shape, const Problem& p, hipStream_t s);
hipError_t launch_mfma_split_tn(Shape shape, const Problem& p, int64_t k_split, float* ws,
                                hipStream_t s);
hipError_t launch_mfma_split_nt(Shape shape, const Problem& p, int64_t k_split, float* ws,
                                hipStream_t s);
hipError_t launch_mfma_split_tt(Shape shape, const Problem& p, int64_t k_split, float* ws,
                                hipStream_t s);
// Where split K's workspace comes from: the library's stream-ordered pool
// (every entry point but one), or the library's fixed device array
// (hip_sgemm_ex_noalloc, for callers that cannot allocate).
enum class Workspace { kPool, kStatic };
// The whole split-K call: the workspace, the split tile kernel, the
// in-order reduction with the alpha/beta epilogue.  With kStatic, S x M x N
// floats beyond the fixed array's size fail with hipErrorInvalidValue
// before anything is enqueued (the entry point checks it first).
hipError_t launch_splitk(Shape shape, int64_t k_split, const Problem& p, hipStream_t s,
                         Workspace w = Workspace::kPool);
// Bytes of the fixed array (SGEMM_NOALLOC_WORKSPACE_BYTES).
int64_t static_workspace_bytes();
// The same split-K call with the split tile kernel given as a function
// (workspace from the pool): the tile catalogue's entries.
using SplitLaunchFn = hipError_t (*)(const Problem&, int64_t k_split, float* ws, hipStream_t);
hipError_t launch_splitk_fn(SplitLaunchFn fn, int64_t k_split, const Problem& p, hipStream_t s);

// The tile catalogue (l9_catalogue.h): legal configurations of level 9's
// tile template for tuning sweeps, row-major operands.  launch runs the
// tile over the whole problem, split over K slices of k_split (raw sums
// into ws, as launch_mfma_split).
struct CatalogueEntry {
  const char* name;
  int bk;
  hipError_t (*launch)(const Problem&, hipStream_t);
  SplitLaunchFn split;
};
// the two halves of the catalogue (entries, with their number in *count)
const CatalogueEntry* catalogue_first(int* count);
const CatalogueEntry* catalogue_second(int* count);
// k_split for a requested slice count: ceil(K / splits) rounded up to BK.
inline int64_t k_split_for(int64_t K, int64_t splits, int bk) {
  const int64_t per = (K + splits - 1) / splits;
  return (per + bk - 1) / bk * bk;
}

// Thin problems (M or N at most kThin) on the vector ALUs: every output is a
// K-long dot product split over lanes and wavefronts and summed in a fixed
// order (deterministic, no atomics, no workspace).
constexpr int kThin = 16;
Geometry few_rows_geometry(int M, int N, int K);
hipError_t launch_few_rows(const Problem& p, hipStream_t s);  // needs M <= kThin
Geometry few_cols_geometry(int M, int N, int K);
hipError_t launch_few_cols(const Problem& p, hipStream_t s);  // needs N <= kThin
// Small problems on the thin matrix-core kernel: 16-row panels of C, each
// panel's columns in blocks of 16-64, K over sixteen wavefronts per block.
Geometry thin_panels_geometry(int M, int N, int K);
hipError_t launch_thin_panels(const Problem& p, hipStream_t s);  // needs M <= 16 * 65535

// Level 10's plan for a shape (the SGEMM_PLAN_* ids of sgemm.h), how many
// kernels a call enqueues and the split-K workspace it takes, decided on
// the host from M, N, K alone (alpha != 0).
struct PlanInfo {
  int plan;
  int launches;
  int64_t workspace_bytes;
};
PlanInfo plan10(int M, int N, int K);
// Level 10's launch with split K's workspace from the given source.
hipError_t launch10_with(const Problem& p, hipStream_t s, Workspace w);

// The rungs (host-side descriptors).
const LevelDesc* level0();
const LevelDesc* level1();
const LevelDesc* level2();
const LevelDesc* level3();
const LevelDesc* level4();
const LevelDesc* level5();
const LevelDesc* level6();
const LevelDesc* level7();
const LevelDesc* level8();
const LevelDesc* level9();
const LevelDesc* level10();

}  // namespace sgemm
