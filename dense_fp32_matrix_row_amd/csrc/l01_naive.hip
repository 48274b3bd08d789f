// l01_naive.hip -- levels 0 and 1: one output element per thread, the dot
// product read straight from HBM/L2 with no on-chip reuse.
//
// Level 0 re-creates [SIX] K1 (section "错在哪一个字"): consecutive lanes of a
// wavefront take consecutive ROWS of C, so one load instruction of the
// wavefront touches 64 different rows of A (64 separate cache lines) while
// its B load is a broadcast.  Level 1 re-creates [SIX] K2 / [L04] section 1.1:
// consecutive lanes take consecutive COLUMNS, so the wavefront's B load is
// one contiguous 256-byte run and its A load a broadcast.  [SIX]'s 4096 vs
// 4097 table shows the level-0 penalty is partly a power-of-two stride effect.
//
// Both accumulate with one fused multiply-add per k in ascending k, so the two
// levels (and level 2) produce identical bits for the same inputs.
#include "sgemm_internal.h"

namespace sgemm {
namespace {

constexpr int kThreads = 256;  // 4 wavefronts of 64 lanes

// Level 0: a block covers 64 rows x 4 columns; lane -> row.
__global__ __launch_bounds__(kThreads) void k_level0(Problem p, int64_t tiles_m,
                                                     int64_t ntiles) {
  const int lane = threadIdx.x % 64;
  const int wave = threadIdx.x / 64;
  for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
    const int64_t row = (t % tiles_m) * 64 + lane;
    const int64_t col = (t / tiles_m) * 4 + wave;
    if (row < p.M && col < p.N) {
      const float* a = p.A + row * p.lda;
      const float* b = p.B + col;
      float acc = 0.0f;
      for (int k = 0; k < p.K; ++k) acc = fmaf(a[k], b[k * p.ldb], acc);
      float* c = p.C + row * p.ldc + col;
      *c = epilogue(acc, p.alpha, p.beta, c);
    }
  }
}

// Level 1: a block covers 4 rows x 64 columns; lane -> column.
__global__ __launch_bounds__(kThreads) void k_level1(Problem p, int64_t tiles_n,
                                                     int64_t ntiles) {
  const int lane = threadIdx.x % 64;
  const int wave = threadIdx.x / 64;
  for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
    const int64_t row = (t / tiles_n) * 4 + wave;
    const int64_t col = (t % tiles_n) * 64 + lane;
    if (row < p.M && col < p.N) {
      const float* a = p.A + row * p.lda;
      const float* b = p.B + col;
      float acc = 0.0f;
      for (int k = 0; k < p.K; ++k) acc = fmaf(a[k], b[k * p.ldb], acc);
      float* c = p.C + row * p.ldc + col;
      *c = epilogue(acc, p.alpha, p.beta, c);
    }
  }
}

Geometry geometry0(int M, int N, int K) {
  return make_geometry(M, N, K, 64, 4, 1, kThreads);
}
Geometry geometry1(int M, int N, int K) {
  return make_geometry(M, N, K, 4, 64, 1, kThreads);
}

hipError_t launch0(const Problem& p, hipStream_t s) {
  const Geometry g = geometry0(p.M, p.N, p.K);
  hipLaunchKernelGGL(k_level0, dim3(static_cast<unsigned>(g.workgroups)),
                     dim3(kThreads), 0, s, p, ceil_div(p.M, 64), g.tiles);
  return hipGetLastError();
}
hipError_t launch1(const Problem& p, hipStream_t s) {
  const Geometry g = geometry1(p.M, p.N, p.K);
  hipLaunchKernelGGL(k_level1, dim3(static_cast<unsigned>(g.workgroups)),
                     dim3(kThreads), 0, s, p, ceil_div(p.N, 64), g.tiles);
  return hipGetLastError();
}

}  // namespace

const LevelDesc* level0() {
  static const LevelDesc d = {"L0_naive_lane_row", geometry0, launch0};
  return &d;
}
const LevelDesc* level1() {
  static const LevelDesc d = {"L1_coalesced_lane_col", geometry1, launch1};
  return &d;
}

}  // namespace sgemm
