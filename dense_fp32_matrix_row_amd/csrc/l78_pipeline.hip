// l78_pipeline.hip -- levels 7 and 8: the level-6 kernel on a double-buffered
// LDS pipeline (level 7), then with wave tiling (level 8).
//
// Level 7 follows [CP04] double_buffer_gemm ("双缓冲流水线"): two LDS
// buffers alternate per K step; the global loads of step k+1 are issued into
// registers before the FMAs of step k, and stored into the other buffer
// after them, so the HBM/L2 latency overlaps the arithmetic and one barrier
// per step suffices: a buffer is rewritten only after the barrier that ends
// every wavefront's reads of it.  BK = 8 with the two buffers unrolled so
// every LDS address is a base plus an immediate.  At 4096^3 four resident
// blocks per CU already overlap one block's loads with the others' FMAs, so
// the double buffer gains 2 % over level 6 there (88.5 against 86.5
// TFLOP/s); at 2048^3, one block per CU, 22 % (45.5 against 37.4).  A is
// staged transposed with rows padded to 132 words.
//
// Level 8 follows [GEMM2]'s warp-tiling section ("三级分块：block → warp →
// thread") on wave64: the 128 x 128 block tile is split 2 x 2 into 64 x 64
// wave tiles and each lane of a wave owns a 2 x 2 grid of 4 x 4 sub-tiles
// (rows wm*64 + i*32 + lr*4 + 0..3, cols wn*64 + j*32 + lc*4 + 0..3 with
// lr = lane%8, lc = lane/8): a wave's reads per k are 64 A and 64 B values
// of LDS (level 7's wave reads 32 A and all 128 B), each 128-bit read
// covering 8 distinct 16-byte groups (128 contiguous bytes) with the other
// lanes broadcast.  [GEMM2]'s thread-swizzling section then re-orders the
// blocks for L2 reuse and reports no gain where the L2 already hits 80 %;
// on MI355X, whose 8 XCDs each have their own L2, an XCD-contiguous order
// (each XCD a contiguous range of tiles, with or without groups of 4-16
// tile rows) measured 3-4 % slower than the plain order for this rung at
// 4096^3 (88.0 against 91.6 TFLOP/s; equal at 2048^3), so level 8 keeps the
// plain order; the matrix-core rungs, whose K steps are far shorter in
// time, use the XCD-contiguous grouped order (l9_tile.h, l10_kloop.hip).
//
// Level 7 and 8 keep their fragment reads and FMAs in program order per k
// (see step below), so both fit 128 VGPRs, four wavefronts per SIMD like
// level 6; both keep one fused multiply-add chain per output in ascending
// k, so they reproduce the bits of levels 0-6.
#include <type_traits>

#include "sgemm_internal.h"

namespace sgemm {
namespace {

constexpr int kBM = 128, kBN = 128, kBK = 8, kTM = 8, kTN = 8;
constexpr int kThreads = 256;
constexpr int kLdaT = kBM + 4;  // transposed-A row stride in LDS (words)
constexpr int kStageIters = (kBM * kBK / 4) / kThreads;  // 1 float4 of A and of B

struct Staged {
  float4 a[kStageIters];
  float4 b[kStageIters];
};

__device__ __forceinline__ void load_stage(Staged& r, const Problem& p,
                                           int64_t row0, int64_t col0,
                                           int64_t k0, int tid) {
#pragma unroll
  for (int s = 0; s < kStageIters; ++s) {
    const int idx = tid + s * kThreads;
    const int a_r = idx / (kBK / 4), a_kq = idx % (kBK / 4);
    r.a[s] = load4(p.A + (row0 + a_r) * p.lda, k0 + 4 * a_kq, p.K,
                        row0 + a_r < p.M);
    const int b_r = idx / (kBN / 4), b_nq = idx % (kBN / 4);
    r.b[s] = load4(p.B + (k0 + b_r) * p.ldb, col0 + 4 * b_nq, p.N,
                        k0 + b_r < p.K);
  }
}

__device__ __forceinline__ void store_stage(const Staged& r,
                                            float (*As)[kLdaT],
                                            float (*Bs)[kBN], int tid) {
#pragma unroll
  for (int s = 0; s < kStageIters; ++s) {
    const int idx = tid + s * kThreads;
    const int a_r = idx / (kBK / 4), a_kq = idx % (kBK / 4);
    As[4 * a_kq + 0][a_r] = r.a[s].x;
    As[4 * a_kq + 1][a_r] = r.a[s].y;
    As[4 * a_kq + 2][a_r] = r.a[s].z;
    As[4 * a_kq + 3][a_r] = r.a[s].w;
    const int b_r = idx / (kBN / 4), b_nq = idx % (kBN / 4);
    *reinterpret_cast<float4*>(&Bs[b_r][4 * b_nq]) = r.b[s];
  }
}

// Thread -> outputs.  Level 7 (as level 6): thread (tr, tc) of a 16 x 16
// grid owns rows 4 tr .. 4 tr + 3 and 64 + 4 tr .., columns 4 tc .. 4 tc + 3
// and 64 + 4 tc .. (the sixteen column-threads' 128-bit B reads then cover
// 256 contiguous bytes, with no bank shared).  Level 8: the wave-tiled map
// above.  m_off(h) / n_off(h) give the tile offset of the h-th group of 4
// rows / cols.
struct MapHalves {
  int m_base, n_base;
  __device__ MapHalves(int tid) : m_base(4 * (tid / 16)), n_base(4 * (tid % 16)) {}
  __device__ int m_off(int h) const { return m_base + (kBM / 2) * h; }
  __device__ int n_off(int h) const { return n_base + (kBN / 2) * h; }
};
struct MapWaveTiled {
  int m_base, n_base;
  __device__ MapWaveTiled(int tid) {
    const int wave = tid / 64, lane = tid % 64;
    m_base = (wave / 2) * 64 + (lane % 8) * 4;
    n_base = (wave % 2) * 64 + (lane / 8) * 4;
  }
  __device__ int m_off(int h) const { return m_base + 32 * h; }
  __device__ int n_off(int h) const { return n_base + 32 * h; }
};

template <class Map>
__device__ __forceinline__ void pipeline_tiles(const Problem& p, int64_t tiles_n,
                                               int64_t ntiles) {
  __shared__ __align__(16) float As[2][kBK][kLdaT];
  __shared__ __align__(16) float Bs[2][kBK][kBN];
  const int tid = threadIdx.x;
  const Map map(tid);
  const int64_t nk = ceil_div(p.K, kBK);
  for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
    const int64_t row0 = (t / tiles_n) * kBM, col0 = (t % tiles_n) * kBN;

    float acc[kTM][kTN];
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
      for (int j = 0; j < kTN; ++j) acc[i][j] = 0.0f;

    Staged st;
    load_stage(st, p, row0, col0, 0, tid);
    store_stage(st, As[0], Bs[0], tid);
    __syncthreads();
    // One K step on LDS buffer CUR (a constant in each use below, so every
    // LDS address is a base plus an immediate): the next step's global
    // loads are issued first, its stores into the other buffer follow the
    // FMAs, one barrier ends the step.
    auto step = [&](auto cur_c, int64_t kt) {
      constexpr int cur = decltype(cur_c)::value;
      const bool more = kt + 1 < nk;
      if (more) load_stage(st, p, row0, col0, (kt + 1) * kBK, tid);
#pragma unroll
      for (int k = 0; k < kBK; ++k) {
        const float4 m0 = *reinterpret_cast<const float4*>(&As[cur][k][map.m_off(0)]);
        const float4 m1 = *reinterpret_cast<const float4*>(&As[cur][k][map.m_off(1)]);
        const float4 n0 = *reinterpret_cast<const float4*>(&Bs[cur][k][map.n_off(0)]);
        const float4 n1 = *reinterpret_cast<const float4*>(&Bs[cur][k][map.n_off(1)]);
        const float regM[kTM] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
        const float regN[kTN] = {n0.x, n0.y, n0.z, n0.w, n1.x, n1.y, n1.z, n1.w};
#pragma unroll
        for (int i = 0; i < kTM; ++i)
#pragma unroll
          for (int j = 0; j < kTN; ++j)
            acc[i][j] = fmaf(regM[i], regN[j], acc[i][j]);
        // Each k's FMAs are issued before the next k's fragment reads and,
        // after the last k, before the stores and the barrier: left free,
        // the compiler hoists a step's 32 reads to its start or sinks its
        // FMAs past the barrier, and either way the fragments hold up to
        // 128 registers -- three wavefronts per SIMD instead of four.
#pragma unroll
        for (int i = 0; i < kTM; ++i)
#pragma unroll
          for (int j = 0; j < kTN; ++j) asm volatile("" : "+v"(acc[i][j])::"memory");
      }
      if (more) store_stage(st, As[cur ^ 1], Bs[cur ^ 1], tid);
      __syncthreads();
    };
    int64_t kt = 0;
    for (; kt + 1 < nk; kt += 2) {
      step(std::integral_constant<int, 0>(), kt);
      step(std::integral_constant<int, 1>(), kt + 1);
    }
    if (kt < nk) step(std::integral_constant<int, 0>(), kt);

#pragma unroll
    for (int i = 0; i < kTM; ++i) {
      const int64_t row = row0 + map.m_off(i / 4) + (i % 4);
      if (row >= p.M) continue;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int64_t col = col0 + map.n_off(h);
        store4(p.C + row * p.ldc + col, col, p.N,
                    make_float4(acc[i][4 * h + 0], acc[i][4 * h + 1],
                                acc[i][4 * h + 2], acc[i][4 * h + 3]),
                    p.alpha, p.beta);
      }
    }
  }
}

// 256 threads, at least four wavefronts per SIMD: 128 VGPRs (a few
// per-tile values spill to scratch outside the K loop)
__global__ __launch_bounds__(kThreads, 4) void k_level7(Problem p, int64_t tiles_n,
                                                        int64_t ntiles) {
  pipeline_tiles<MapHalves>(p, tiles_n, ntiles);
}

__global__ __launch_bounds__(kThreads, 4) void k_level8(Problem p, int64_t tiles_n,
                                                        int64_t ntiles) {
  pipeline_tiles<MapWaveTiled>(p, tiles_n, ntiles);
}

Geometry geometry78(int M, int N, int K) {
  return make_geometry(M, N, K, kBM, kBN, kBK, kThreads);
}

hipError_t launch7(const Problem& p, hipStream_t s) {
  const Geometry g = geometry78(p.M, p.N, p.K);
  hipLaunchKernelGGL(k_level7, dim3(static_cast<unsigned>(g.workgroups)), dim3(kThreads), 0, s,
                     p, ceil_div(p.N, kBN), g.tiles);
  return hipGetLastError();
}

hipError_t launch8(const Problem& p, hipStream_t s) {
  const Geometry g = geometry78(p.M, p.N, p.K);
  hipLaunchKernelGGL(k_level8, dim3(static_cast<unsigned>(g.workgroups)), dim3(kThreads), 0, s,
                     p, ceil_div(p.N, kBN), g.tiles);
  return hipGetLastError();
}

}  // namespace

const LevelDesc* level7() {
  static const LevelDesc d = {"L7_double_buffer", geometry78, launch7};
  return &d;
}
const LevelDesc* level8() {
  static const LevelDesc d = {"L8_wave_tile", geometry78, launch8};
  return &d;
}

}  // namespace sgemm
