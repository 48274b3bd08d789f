// l56_regtile2d.hip -- levels 5 and 6: 2-D register tiles, a 128 x 128 C tile
// per 256-thread block and an 8 x 8 outer product per thread.
//
// Level 5 re-designs [SIX] K5, [CP04] register_tiling_gemm (BM = BN = 128,
// BK = 8, TM = TN = 8: 64 accumulators + 8 + 8 fragment registers) and
// [GEMM2] kernel 5 for wave64: per k a thread reads 8 A values and 8 B values
// from LDS and issues 64 FMAs ("square beats strip", [GEMM2]).  Loads are
// element-wise and cooperative (each thread stages 4 A and 4 B elements per
// phase); A stays row-major in LDS with rows padded to BK+1 words so the
// four row groups a wavefront reads fall in different banks.  Bank
// arithmetic on wave64 (LDS bank = word mod 64; a 32-bit access is served
// per half-wavefront): a thread's eight columns are tc, tc + 16, ...,
// tc + 112 rather than eight adjacent ones, so the sixteen column-threads of
// a B read touch sixteen adjacent words (adjacent columns would put them
// 8 words apart, two per bank); and each half-wavefront of the A stage
// stores rows 8 apart (rows g, g+8, g+16, g+24 x 8 k: 9-word rows put them
// on 32 different banks, where four adjacent rows wrap onto each other).
//
// Level 6 adds the two changes of [SIX] K6 and [GEMM2] kernel 6: A is stored
// TRANSPOSED in LDS (As[k][m]) so a thread's 8 M-direction values are
// contiguous and come in as two 128-bit LDS reads (B's already are), and the
// global loads and the C epilogue move 128 bits per lane.  On gfx950 a
// 128-bit global access needs only 4-byte alignment, so the vector path runs
// for any row stride; partial groups at the K and N edges are element-wise,
// never dropped.  The transposed rows are
// padded to 132 words, which puts the two k-groups of a half-wavefront's
// transposing 32-bit stores 16 banks apart (136 words overlaid them), and a
// thread's eight columns are two groups of four 64 apart (4 tc .. 4 tc + 3
// and 64 + 4 tc ..), so the sixteen column-threads' 128-bit B reads cover
// 256 contiguous bytes (adjacent groups of eight would leave 16-byte gaps
// and two threads per bank).
//
// Both accumulate each output as one fused multiply-add chain in ascending k,
// so they reproduce the bits of levels 0-4.
#include "sgemm_internal.h"

namespace sgemm {
namespace {

constexpr int kBM = 128, kBN = 128, kBK = 8, kTM = 8, kTN = 8;
constexpr int kThreads = (kBM / kTM) * (kBN / kTN);  // 256
constexpr int kTcols = kBN / kTN;                     // 16 threads across N

// At least four wavefronts per SIMD (128 VGPRs; a few per-tile addresses
// spill to scratch): with the reads kept per k, 4096^3 runs at 75.6 TFLOP/s
// against 47.3 at 204 VGPRs and two wavefronts per SIMD.
__global__ __launch_bounds__(kThreads, 4) void k_level5(Problem p, int64_t tiles_n,
                                                     int64_t ntiles) {
  __shared__ float As[kBM][kBK + 1];
  __shared__ float Bs[kBK][kBN];
  const int tid = threadIdx.x;
  const int tr = tid / kTcols, tc = tid % kTcols;
  for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
    const int64_t row0 = (t / tiles_n) * kBM;
    const int64_t col0 = (t % tiles_n) * kBN;
    float acc[kTM][kTN];
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
      for (int j = 0; j < kTN; ++j) acc[i][j] = 0.0f;
    for (int64_t k0 = 0; k0 < p.K; k0 += kBK) {
#pragma unroll
      for (int s = 0; s < (kBM * kBK) / kThreads; ++s) {
        // half-wavefront g = tid / 32 stores rows g + 8q + 32s (q = 0..3)
        const int c = tid % kBK, r = tid / 32 + 8 * ((tid % 32) / kBK) + 32 * s;
        As[r][c] = (row0 + r < p.M && k0 + c < p.K)
                       ? p.A[(row0 + r) * p.lda + k0 + c]
                       : 0.0f;
      }
#pragma unroll
      for (int s = 0; s < (kBK * kBN) / kThreads; ++s) {
        const int idx = tid + s * kThreads;
        const int r = idx / kBN, c = idx % kBN;
        Bs[r][c] = (k0 + r < p.K && col0 + c < p.N)
                       ? p.B[(k0 + r) * p.ldb + col0 + c]
                       : 0.0f;
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < kBK; ++k) {
        float regM[kTM], regN[kTN];
#pragma unroll
        for (int i = 0; i < kTM; ++i) regM[i] = As[tr * kTM + i][k];
#pragma unroll
        for (int j = 0; j < kTN; ++j) regN[j] = Bs[k][tc + kTcols * j];
#pragma unroll
        for (int i = 0; i < kTM; ++i)
#pragma unroll
          for (int j = 0; j < kTN; ++j)
            acc[i][j] = fmaf(regM[i], regN[j], acc[i][j]);
        // each k's FMAs before the next k's reads: left free, the compiler
        // hoists all eight k's 128 scalar reads to the top of the phase
#pragma unroll
        for (int i = 0; i < kTM; ++i)
#pragma unroll
          for (int j = 0; j < kTN; ++j) asm volatile("" : "+v"(acc[i][j])::"memory");
      }
      __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < kTM; ++i) {
      const int64_t row = row0 + tr * kTM + i;
      if (row >= p.M) continue;
#pragma unroll
      for (int j = 0; j < kTN; ++j) {
        const int64_t col = col0 + tc + kTcols * j;
        if (col < p.N) {
          float* c = p.C + row * p.ldc + col;
          *c = epilogue(acc[i][j], p.alpha, p.beta, c);
        }
      }
    }
  }
}

constexpr int kLdaT = kBM + 4;  // transposed-A row stride in LDS (words)

__global__ __launch_bounds__(kThreads) void k_level6(Problem p, int64_t tiles_n,
                                                     int64_t ntiles) {
  __shared__ __align__(16) float As[kBK][kLdaT];
  __shared__ __align__(16) float Bs[kBK][kBN];
  const int tid = threadIdx.x;
  const int tr = tid / kTcols, tc = tid % kTcols;
  // one 4-wide group of A (row a_r, k-group a_kq) and one of B per phase
  const int a_r = tid / (kBK / 4), a_kq = tid % (kBK / 4);
  const int b_r = tid / (kBN / 4), b_nq = tid % (kBN / 4);
  for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
    const int64_t row0 = (t / tiles_n) * kBM;
    const int64_t col0 = (t % tiles_n) * kBN;
    float acc[kTM][kTN];
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
      for (int j = 0; j < kTN; ++j) acc[i][j] = 0.0f;
    const float* a_row = p.A + (row0 + a_r) * p.lda;
    const bool a_ok = row0 + a_r < p.M;
    for (int64_t k0 = 0; k0 < p.K; k0 += kBK) {
      const float4 va = load4(a_row, k0 + 4 * a_kq, p.K, a_ok);
      As[4 * a_kq + 0][a_r] = va.x;
      As[4 * a_kq + 1][a_r] = va.y;
      As[4 * a_kq + 2][a_r] = va.z;
      As[4 * a_kq + 3][a_r] = va.w;
      const float4 vb = load4(p.B + (k0 + b_r) * p.ldb, col0 + 4 * b_nq,
                                   p.N, k0 + b_r < p.K);
      *reinterpret_cast<float4*>(&Bs[b_r][4 * b_nq]) = vb;
      __syncthreads();
#pragma unroll
      for (int k = 0; k < kBK; ++k) {
        const float4 m0 = *reinterpret_cast<const float4*>(&As[k][tr * kTM]);
        const float4 m1 = *reinterpret_cast<const float4*>(&As[k][tr * kTM + 4]);
        const float4 n0 = *reinterpret_cast<const float4*>(&Bs[k][4 * tc]);
        const float4 n1 = *reinterpret_cast<const float4*>(&Bs[k][kBN / 2 + 4 * tc]);
        const float regM[kTM] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
        const float regN[kTN] = {n0.x, n0.y, n0.z, n0.w, n1.x, n1.y, n1.z, n1.w};
#pragma unroll
        for (int i = 0; i < kTM; ++i)
#pragma unroll
          for (int j = 0; j < kTN; ++j)
            acc[i][j] = fmaf(regM[i], regN[j], acc[i][j]);
      }
      __syncthreads();
    }
    const int64_t col = col0 + 4 * tc, col_hi = col + kBN / 2;
#pragma unroll
    for (int i = 0; i < kTM; ++i) {
      const int64_t row = row0 + tr * kTM + i;
      if (row >= p.M) continue;
      float* c = p.C + row * p.ldc;
      store4(c + col, col, p.N,
                  make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]),
                  p.alpha, p.beta);
      store4(c + col_hi, col_hi, p.N,
                  make_float4(acc[i][4], acc[i][5], acc[i][6], acc[i][7]),
                  p.alpha, p.beta);
    }
  }
}

Geometry geometry56(int M, int N, int K) {
  return make_geometry(M, N, K, kBM, kBN, kBK, kThreads);
}

hipError_t launch5(const Problem& p, hipStream_t s) {
  const Geometry g = geometry56(p.M, p.N, p.K);
  hipLaunchKernelGGL(k_level5, dim3(static_cast<unsigned>(g.workgroups)),
                     dim3(kThreads), 0, s, p, ceil_div(p.N, kBN), g.tiles);
  return hipGetLastError();
}

hipError_t launch6(const Problem& p, hipStream_t s) {
  const Geometry g = geometry56(p.M, p.N, p.K);
  hipLaunchKernelGGL(k_level6, dim3(static_cast<unsigned>(g.workgroups)),
                     dim3(kThreads), 0, s, p, ceil_div(p.N, kBN), g.tiles);
  return hipGetLastError();
}

}  // namespace

const LevelDesc* level5() {
  static const LevelDesc d = {"L5_regtile_2d_8x8", geometry56, launch5};
  return &d;
}
const LevelDesc* level6() {
  static const LevelDesc d = {"L6_vec4_transposed_a", geometry56, launch6};
  return &d;
}

}  // namespace sgemm
