// l4_regtile1d.hip -- level 4: 1-D register tile, 8 outputs of one column per
// thread.
//
// Re-designs [SIX] K4 ("复用从哪来": one B element held in a register and
// used for 8 outputs of the same column) and [GEMM2] kernel 4 (BM = BN = 64,
// BK = 8, TM = 8, 512 threads) for wave64: wavefront w of the 8 owns rows
// 8w .. 8w+7 of the 64 x 64 C tile and its 64 lanes own the 64 columns, so a
// B-tile read Bs[k][lane] is one conflict-free 256-byte LDS access and each
// A-tile read As[8w+i][k] is a single word broadcast to the whole wavefront.
// Per k a lane issues 1 B read + 8 broadcast A reads for 8 FMAs.
//
// One fused multiply-add chain per output in ascending k: the bits equal
// those of levels 0-3.
#include "sgemm_internal.h"

namespace sgemm {
namespace {

constexpr int kBM = 64, kBN = 64, kBK = 8, kTM = 8;
constexpr int kThreads = (kBM / kTM) * kBN;  // 512: 8 wavefronts

__global__ __launch_bounds__(kThreads) void k_level4(Problem p, int64_t tiles_n,
                                                     int64_t ntiles) {
  __shared__ float As[kBM][kBK];
  __shared__ float Bs[kBK][kBN];
  const int tid = threadIdx.x;
  const int lane_col = tid % kBN;  // this lane's column in the tile
  const int rgrp = tid / kBN;      // = wavefront index: rows 8*rgrp ..
  // staging map: one A element and one B element per thread per phase
  const int a_r = tid / kBK, a_c = tid % kBK;
  const int b_r = tid / kBN, b_c = tid % kBN;
  for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
    const int64_t row0 = (t / tiles_n) * kBM;
    const int64_t col0 = (t % tiles_n) * kBN;
    const bool a_row_ok = row0 + a_r < p.M;
    const bool b_col_ok = col0 + b_c < p.N;
    float acc[kTM];
#pragma unroll
    for (int i = 0; i < kTM; ++i) acc[i] = 0.0f;
    for (int64_t k0 = 0; k0 < p.K; k0 += kBK) {
      As[a_r][a_c] = (a_row_ok && k0 + a_c < p.K)
                         ? p.A[(row0 + a_r) * p.lda + k0 + a_c]
                         : 0.0f;
      Bs[b_r][b_c] = (k0 + b_r < p.K && b_col_ok)
                         ? p.B[(k0 + b_r) * p.ldb + col0 + b_c]
                         : 0.0f;
      __syncthreads();
#pragma unroll
      for (int k = 0; k < kBK; ++k) {
        const float b = Bs[k][lane_col];
#pragma unroll
        for (int i = 0; i < kTM; ++i)
          acc[i] = fmaf(As[rgrp * kTM + i][k], b, acc[i]);
      }
      __syncthreads();
    }
    const int64_t col = col0 + lane_col;
    if (col < p.N) {
#pragma unroll
      for (int i = 0; i < kTM; ++i) {
        const int64_t row = row0 + rgrp * kTM + i;
        if (row < p.M) {
          float* c = p.C + row * p.ldc + col;
          *c = epilogue(acc[i], p.alpha, p.beta, c);
        }
      }
    }
  }
}

Geometry geometry4(int M, int N, int K) {
  return make_geometry(M, N, K, kBM, kBN, kBK, kThreads);
}

hipError_t launch4(const Problem& p, hipStream_t s) {
  const Geometry g = geometry4(p.M, p.N, p.K);
  hipLaunchKernelGGL(k_level4, dim3(static_cast<unsigned>(g.workgroups)),
                     dim3(kThreads), 0, s, p, ceil_div(p.N, kBN), g.tiles);
  return hipGetLastError();
}

}  // namespace

const LevelDesc* level4() {
  static const LevelDesc d = {"L4_regtile_1d_8x1", geometry4, launch4};
  return &d;
}

}  // namespace sgemm
