// l23_lds_tile.hip -- levels 2 and 3: LDS tiling, one (level 2) or four
// (level 3) outputs per thread.
//
// Level 2 re-designs [SIX] K3 / [CP04] tiled_gemm / [L04] sections 2.2-2.5
// for wave64: a 32 x 32 C tile per 1024-thread block; per phase the block
// stages a 32 x 32 slab of A (sliding right) and of B (sliding down) in LDS,
// one element per thread, so each element fetched from HBM/L2 is used 32
// times.  Two barriers per phase: after the stores (read-after-write) and
// after the FMAs (write-after-read), [L04] section 2.4.  Boundary rule of
// [L04] section 2.5: the phase count is rounded up, out-of-range elements are
// stored as zero, out-of-range threads stay in every barrier and only the
// final store is guarded.
//
// A wavefront is two rows of 32 lanes (ty, ty+1), so its A-tile read As[ty][k]
// touches two LDS words; the rows are padded to 33 words (the +1 padding of
// [L04] section 3) so the two words sit in different banks.  Its B-tile read
// Bs[k][tx] is the same 32 words for both halves (broadcast).
//
// Level 3 is [SIX] K3c / [CP04] coarse_gemm / [L04] section 2.7: the block
// owns COARSE = 4 neighbouring 32 x 32 tiles of one row band (32 x 128), so the
// A slab of each phase is loaded once and used for four outputs per thread.
//
// Every output is one fused multiply-add chain in ascending k (zero-filled
// terms add +0), so both levels reproduce the bits of levels 0 and 1.
#include "sgemm_internal.h"

namespace sgemm {
namespace {

constexpr int kTile = 32;
constexpr int kThreads = kTile * kTile;  // 1024: 16 wavefronts
constexpr int kCoarse = 4;

__global__ __launch_bounds__(kThreads) void k_level2(Problem p, int64_t tiles_n,
                                                     int64_t ntiles) {
  __shared__ float As[kTile][kTile + 1];
  __shared__ float Bs[kTile][kTile + 1];
  const int tx = threadIdx.x % kTile;
  const int ty = threadIdx.x / kTile;
  for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
    const int64_t row = (t / tiles_n) * kTile + ty;
    const int64_t col = (t % tiles_n) * kTile + tx;
    const bool row_ok = row < p.M, col_ok = col < p.N;
    float acc = 0.0f;
    for (int64_t k0 = 0; k0 < p.K; k0 += kTile) {
      const int64_t ak = k0 + tx, bk = k0 + ty;
      As[ty][tx] = (row_ok && ak < p.K) ? p.A[row * p.lda + ak] : 0.0f;
      Bs[ty][tx] = (bk < p.K && col_ok) ? p.B[bk * p.ldb + col] : 0.0f;
      __syncthreads();
#pragma unroll
      for (int k = 0; k < kTile; ++k) acc = fmaf(As[ty][k], Bs[k][tx], acc);
      __syncthreads();
    }
    if (row_ok && col_ok) {
      float* c = p.C + row * p.ldc + col;
      *c = epilogue(acc, p.alpha, p.beta, c);
    }
  }
}

__global__ __launch_bounds__(kThreads) void k_level3(Problem p, int64_t tiles_n,
                                                     int64_t ntiles) {
  __shared__ float As[kTile][kTile + 1];
  __shared__ float Bs[kTile][kTile * kCoarse];
  const int tx = threadIdx.x % kTile;
  const int ty = threadIdx.x / kTile;
  for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
    const int64_t row = (t / tiles_n) * kTile + ty;
    const int64_t col0 = (t % tiles_n) * (kTile * kCoarse) + tx;
    const bool row_ok = row < p.M;
    float acc[kCoarse];
#pragma unroll
    for (int c = 0; c < kCoarse; ++c) acc[c] = 0.0f;
    for (int64_t k0 = 0; k0 < p.K; k0 += kTile) {
      const int64_t ak = k0 + tx, bk = k0 + ty;
      As[ty][tx] = (row_ok && ak < p.K) ? p.A[row * p.lda + ak] : 0.0f;
#pragma unroll
      for (int c = 0; c < kCoarse; ++c) {
        const int64_t col = col0 + c * kTile;
        Bs[ty][tx + c * kTile] =
            (bk < p.K && col < p.N) ? p.B[bk * p.ldb + col] : 0.0f;
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < kTile; ++k) {
        const float a = As[ty][k];
#pragma unroll
        for (int c = 0; c < kCoarse; ++c)
          acc[c] = fmaf(a, Bs[k][tx + c * kTile], acc[c]);
      }
      __syncthreads();
    }
    if (row_ok) {
#pragma unroll
      for (int c = 0; c < kCoarse; ++c) {
        const int64_t col = col0 + c * kTile;
        if (col < p.N) {
          float* cp = p.C + row * p.ldc + col;
          *cp = epilogue(acc[c], p.alpha, p.beta, cp);
        }
      }
    }
  }
}

Geometry geometry2(int M, int N, int K) {
  return make_geometry(M, N, K, kTile, kTile, kTile, kThreads);
}
Geometry geometry3(int M, int N, int K) {
  return make_geometry(M, N, K, kTile, kTile * kCoarse, kTile, kThreads);
}

hipError_t launch2(const Problem& p, hipStream_t s) {
  const Geometry g = geometry2(p.M, p.N, p.K);
  hipLaunchKernelGGL(k_level2, dim3(static_cast<unsigned>(g.workgroups)),
                     dim3(kThreads), 0, s, p, ceil_div(p.N, kTile), g.tiles);
  return hipGetLastError();
}
hipError_t launch3(const Problem& p, hipStream_t s) {
  const Geometry g = geometry3(p.M, p.N, p.K);
  hipLaunchKernelGGL(k_level3, dim3(static_cast<unsigned>(g.workgroups)),
                     dim3(kThreads), 0, s, p, ceil_div(p.N, kTile * kCoarse),
                     g.tiles);
  return hipGetLastError();
}

}  // namespace

const LevelDesc* level2() {
  static const LevelDesc d = {"L2_lds_tile32", geometry2, launch2};
  return &d;
}
const LevelDesc* level3() {
  static const LevelDesc d = {"L3_coarsen_1x4", geometry3, launch3};
  return &d;
}

}  // namespace sgemm
