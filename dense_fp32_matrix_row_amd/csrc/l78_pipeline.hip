// l78_pipeline.hip -- levels 7 and 8: the level-6 kernel on a double-buffered
// LDS pipeline (level 7), then with wave tiling and an XCD-aware block order
// (level 8).
//
// Level 7 follows [CP04] double_buffer_gemm ("双缓冲流水线"): two LDS
// buffers alternate per K step; the global loads of step k+1 are issued into
// registers before the FMAs of step k, and stored into the other buffer
// after them, so the HBM/L2 latency overlaps the arithmetic and one barrier
// per step suffices: a buffer is rewritten only after the barrier that ends
// every wavefront's reads of it.  BK = 8 and the k loop unrolled by 4 keep
// the kernel at 118 VGPRs, four wavefronts per SIMD like level 6 (BK = 16
// needed 140, three per SIMD, and ran 3.5 % slower at 4096^3).  On MI355X the
// double buffer gains little over level 6: four resident blocks per CU
// already overlap one block's loads with the others' FMAs, which is what the
// double buffer buys a single block.  A is staged transposed with rows padded
// to 132 words.
//
// Level 8 follows [GEMM2]'s warp-tiling section ("三级分块：block → warp →
// thread") on wave64: the 128 x 128 block tile is split 2 x 2 into 64 x 64
// wave tiles and each lane of a wave owns a 2 x 2 grid of 4 x 4 sub-tiles
// (rows wm*64 + i*32 + lr*4 + 0..3, cols wn*64 + j*32 + lc*4 + 0..3 with
// lr = lane/8, lc = lane%8).  Its four 128-bit LDS reads per k then cover 8
// distinct 16-byte groups (128 contiguous bytes) per wavefront, with the other
// lanes broadcast, and its C stores are 128-byte rows.  Blocks are re-ordered
// twice ([GEMM2] "thread swizzling" section; on MI355X the point is the eight
// separate L2s): the hardware hands consecutive block ids round-robin to the
// 8 XCDs, so each XCD first receives a contiguous range of logical tile ids,
// and logical ids walk C in groups of 8 tile-rows so that concurrently
// resident tiles share A row panels and B column panels inside one L2.
//
// Both keep one fused multiply-add chain per output in ascending k, so they
// reproduce the bits of levels 0-6.
#include "sgemm_internal.h"

namespace sgemm {
namespace {

constexpr int kBM = 128, kBN = 128, kBK = 8, kTM = 8, kTN = 8;
constexpr int kThreads = 256;
constexpr int kLdaT = kBM + 4;  // transposed-A row stride in LDS (words)
constexpr int kGroupM = 8;      // tile-rows per group in the level-8 order
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

// Thread -> outputs.  Level 7: thread (tr, tc) of a 16 x 16 grid owns the
// contiguous 8 x 8 block at (tr*8, tc*8).  Level 8: the wave-tiled map above.
// m_off(h) / n_off(h) give the tile offset of the h-th group of 4 rows / cols.
struct MapContiguous {
  int m_base, n_base;
  __device__ MapContiguous(int tid)
      : m_base((tid / 16) * kTM), n_base((tid % 16) * kTN) {}
  __device__ int m_off(int h) const { return m_base + 4 * h; }
  __device__ int n_off(int h) const { return n_base + 4 * h; }
};
struct MapWaveTiled {
  int m_base, n_base;
  __device__ MapWaveTiled(int tid) {
    const int wave = tid / 64, lane = tid % 64;
    m_base = (wave / 2) * 64 + (lane / 8) * 4;
    n_base = (wave % 2) * 64 + (lane % 8) * 4;
  }
  __device__ int m_off(int h) const { return m_base + 32 * h; }
  __device__ int n_off(int h) const { return n_base + 32 * h; }
};

template <bool SWIZZLE, class Map>
__device__ __forceinline__ void pipeline_tiles(const Problem& p,
                                               int64_t tiles_m,
                                               int64_t tiles_n,
                                               int64_t ntiles) {
  __shared__ __align__(16) float As[2][kBK][kLdaT];
  __shared__ __align__(16) float Bs[2][kBK][kBN];
  const int tid = threadIdx.x;
  const Map map(tid);
  const int64_t nk = ceil_div(p.K, kBK);
  const int64_t first =
      SWIZZLE ? xcd_contiguous(blockIdx.x, gridDim.x) : int64_t(blockIdx.x);
  for (int64_t t = first; t < ntiles; t += gridDim.x) {
    int64_t tm, tn;
    if (SWIZZLE) {
      const int64_t group = kGroupM * tiles_n;
      const int64_t first_m = (t / group) * kGroupM;
      const int64_t gm = tiles_m - first_m < kGroupM ? tiles_m - first_m : kGroupM;
      const int64_t in = t % group;
      tm = first_m + in % gm;
      tn = in / gm;
    } else {
      tm = t / tiles_n;
      tn = t % tiles_n;
    }
    const int64_t row0 = tm * kBM, col0 = tn * kBN;

    float acc[kTM][kTN];
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
      for (int j = 0; j < kTN; ++j) acc[i][j] = 0.0f;

    Staged st;
    load_stage(st, p, row0, col0, 0, tid);
    store_stage(st, As[0], Bs[0], tid);
    __syncthreads();
    for (int64_t kt = 0; kt < nk; ++kt) {
      const int cur = static_cast<int>(kt & 1);
      const bool more = kt + 1 < nk;
      if (more) load_stage(st, p, row0, col0, (kt + 1) * kBK, tid);
      // Unrolled by 4: fully unrolled, the compiler hoists every k-step's
      // fragment reads above the loop (233 VGPRs, two wavefronts per SIMD).
#pragma unroll 4
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
      }
      if (more) store_stage(st, As[cur ^ 1], Bs[cur ^ 1], tid);
      __syncthreads();
    }

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

__global__ __launch_bounds__(kThreads) void k_level7(Problem p, int64_t tiles_m,
                                                     int64_t tiles_n,
                                                     int64_t ntiles) {
  pipeline_tiles<false, MapContiguous>(p, tiles_m, tiles_n, ntiles);
}

__global__ __launch_bounds__(kThreads) void k_level8(Problem p, int64_t tiles_m,
                                                     int64_t tiles_n,
                                                     int64_t ntiles) {
  pipeline_tiles<true, MapWaveTiled>(p, tiles_m, tiles_n, ntiles);
}

Geometry geometry78(int M, int N, int K) {
  return make_geometry(M, N, K, kBM, kBN, kBK, kThreads);
}

hipError_t launch7(const Problem& p, hipStream_t s) {
  const Geometry g = geometry78(p.M, p.N, p.K);
  const dim3 grid(static_cast<unsigned>(g.workgroups)), block(kThreads);
  const int64_t tm = ceil_div(p.M, kBM), tn = ceil_div(p.N, kBN);
  hipLaunchKernelGGL(k_level7, grid, block, 0, s, p, tm, tn, g.tiles);
  return hipGetLastError();
}

hipError_t launch8(const Problem& p, hipStream_t s) {
  const Geometry g = geometry78(p.M, p.N, p.K);
  const dim3 grid(static_cast<unsigned>(g.workgroups)), block(kThreads);
  const int64_t tm = ceil_div(p.M, kBM), tn = ceil_div(p.N, kBN);
  hipLaunchKernelGGL(k_level8, grid, block, 0, s, p, tm, tn, g.tiles);
  return hipGetLastError();
}

}  // namespace

const LevelDesc* level7() {
  static const LevelDesc d = {"L7_double_buffer", geometry78, launch7};
  return &d;
}
const LevelDesc* level8() {
  static const LevelDesc d = {"L8_wave_tile_xcd_swizzle", geometry78, launch8};
  return &d;
}

}  // namespace sgemm
