// l10_thin.hip -- the thin-problem kernels of the dispatching rung: C blocks
// with at most kThin (16) rows or at most kThin columns, on the vector ALUs.
//
// A thin product reads one operand in full and does little arithmetic per
// byte (M = 1 is a matrix-vector product), so it is HBM-bound; a matrix-core
// tile would leave most of its 32 x 32 blocks empty.  The pages' answer for
// a row panel is one lane per output column with the K loop inside ([SIX]
// K1-K2); a single M = 1 row of 4097 columns gives only 4097 lanes, far from
// filling 256 CUs, so here each output's K sum is split over the lanes and
// wavefronts of one block instead and combined in a fixed order:
//   - per lane, a float32 FMA chain over its own k values (ascending);
//   - across lanes, an xor butterfly (partner order fixed by lane bits);
//   - across wavefronts, an in-order sum through LDS.
// The order depends only on the shape, never on timing: results are
// bit-reproducible, with no atomics and no workspace.
//
// Used for problems with M <= 16 or N <= 16, and for the one- to
// sixteen-row/column fringe left beside the matrix-core tiles of large
// ragged problems (4097^3: a 4096 x 4096 tile grid plus a 1-row and a
// 1-column fringe).
#include "sgemm_internal.h"

namespace sgemm {
namespace {

__device__ __forceinline__ float fget(const float4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// ---------------------------------------------------------------------------
// Few rows: M <= RP.  Block b owns columns [16b, 16b + 16).  Lane l of
// wavefront w takes the column quad q = l % 4 (4 adjacent columns, one
// 128-bit B access) and, in each sweep of 64*WAVES k values, the k quad
// g = l / 4 of its wavefront's 64: k = sweep*64*WAVES + 64*w + 4*g .. +3.
// For each such k it reads 4 B rows (4 x 4 floats) and the RP A values of
// those k (one 128-bit access per row of A).
template <int RP>
struct FewRows {
  static constexpr int WAVES = RP <= 4 ? 16 : 8;   // register budget
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int KSWEEP = 64 * WAVES;
};

// TA: A stored K x M (element (r, k) at A[k * lda + r]); TB: B stored N x K
// (element (k, n) at B[n * ldb + k]: the lane's four columns come as four
// 128-bit reads along k and are transposed in registers).
template <int RP, bool TA, bool TB>
__global__ __launch_bounds__(FewRows<RP>::THREADS) void k_few_rows(Problem p,
                                                                   int64_t nblocks) {
  constexpr int WAVES = FewRows<RP>::WAVES, KSWEEP = FewRows<RP>::KSWEEP;
  __shared__ float red[WAVES][RP][16];
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
  const int q = lane % 4, g = lane / 4;

  // neighbouring column blocks read the two halves of the same 128-byte B
  // lines: keep them on one XCD (one L2)
  for (int64_t blk = xcd_contiguous(blockIdx.x, gridDim.x); blk < nblocks; blk += gridDim.x) {
    const int64_t c0 = blk * 16;
    const int64_t col = c0 + 4 * q;
    float acc[RP][4];
#pragma unroll
    for (int r = 0; r < RP; ++r)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[r][c] = 0.0f;

    for (int64_t k = 64 * wave + 4 * g; k < p.K; k += KSWEEP) {
      float4 b[4];
      if (TB) {
        float4 v[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) v[c] = load4(p.B + (col + c) * p.ldb, k, p.K, col + c < p.N);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          b[j] = make_float4(fget(v[0], j), fget(v[1], j), fget(v[2], j), fget(v[3], j));
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          b[j] = load4(p.B + (k + j) * p.ldb, col, p.N, k + j < p.K);
      }
#pragma unroll
      for (int r = 0; r < RP; ++r) {
        float4 a;
        if (TA) {
          const bool ok = r < p.M;
          a = make_float4(ok && k < p.K ? p.A[k * p.lda + r] : 0.0f,
                          ok && k + 1 < p.K ? p.A[(k + 1) * p.lda + r] : 0.0f,
                          ok && k + 2 < p.K ? p.A[(k + 2) * p.lda + r] : 0.0f,
                          ok && k + 3 < p.K ? p.A[(k + 3) * p.lda + r] : 0.0f);
        } else {
          a = load4(p.A + r * p.lda, k, p.K, r < p.M);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float av = fget(a, j);
          acc[r][0] = fmaf(av, b[j].x, acc[r][0]);
          acc[r][1] = fmaf(av, b[j].y, acc[r][1]);
          acc[r][2] = fmaf(av, b[j].z, acc[r][2]);
          acc[r][3] = fmaf(av, b[j].w, acc[r][3]);
        }
      }
    }

    // Sum over the 16 k quads of the wavefront (lane bits 2-5), then over
    // the wavefronts in order.
#pragma unroll
    for (int r = 0; r < RP; ++r)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        float v = acc[r][c];
        v += __shfl_xor(v, 4);
        v += __shfl_xor(v, 8);
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        if (g == 0) red[wave][r][4 * q + c] = v;
      }
    __syncthreads();
    if (tid < RP * 16) {
      const int r = tid / 16, cc = tid % 16;
      float sum = red[0][r][cc];
#pragma unroll
      for (int w = 1; w < WAVES; ++w) sum += red[w][r][cc];
      if (r < p.M && c0 + cc < p.N) {
        float* c = p.C + r * p.ldc + c0 + cc;
        *c = epilogue(sum, p.alpha, p.beta, c);
      }
    }
    __syncthreads();  // red is rewritten by the next column block
  }
}

// ---------------------------------------------------------------------------
// Few columns: N <= WP.  Block b owns rows [16b, 16b + 16), one row per
// wavefront.  K is walked in chunks of KC: the chunk's WP columns of B are
// staged in LDS column by column (Bs[c][k], so that a lane's four k of one
// column are one conflict-free 128-bit read), and lane l takes the k quads
// 4*l + 256*t of the chunk, reading its A row with 128-bit loads (a
// wavefront reads 1 KB of one A row per instruction).  The next chunk's A
// values are requested before the barrier that guards the B staging, so the
// two latencies overlap.
constexpr int kRowsPerBlock = 16;
constexpr int kColThreads = 64 * kRowsPerBlock;

template <int WP>
struct FewCols {
  static constexpr int KC = WP <= 8 ? 2048 : 1024;  // LDS: 64 KB at most
  static constexpr int QUADS = KC / 256;            // k quads per lane per chunk
};

// TB: B stored N x K (the staged strip is then contiguous along k).  A is
// always row-major here: with A stored K x M a wavefront's row would be a
// strided column, so the dispatcher gives such problems to the tile kernels.
template <int WP, bool TB>
__global__ __launch_bounds__(kColThreads) void k_few_cols(Problem p, int64_t nblocks) {
  constexpr int KC = FewCols<WP>::KC, QUADS = FewCols<WP>::QUADS;
  __shared__ __align__(16) float Bs[WP][KC];
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;

  for (int64_t blk = xcd_contiguous(blockIdx.x, gridDim.x); blk < nblocks; blk += gridDim.x) {
    const int64_t row = blk * kRowsPerBlock + wave;
    const bool has_row = row < p.M;
    const float* arow = p.A + (has_row ? row : 0) * p.lda;
    float acc[WP];
#pragma unroll
    for (int c = 0; c < WP; ++c) acc[c] = 0.0f;

    for (int64_t kc = 0; kc < p.K; kc += KC) {
      float4 a[QUADS];
#pragma unroll
      for (int t = 0; t < QUADS; ++t) a[t] = load4(arow, kc + 4 * lane + 256 * t, p.K, has_row);
      __syncthreads();  // every wavefront is done with the previous chunk
      for (int e = tid; e < WP * KC; e += kColThreads) {
        const int c = e / KC, kk = e % KC;
        const bool ok = kc + kk < p.K && c < p.N;
        Bs[c][kk] = !ok ? 0.0f : TB ? p.B[c * p.ldb + kc + kk] : p.B[(kc + kk) * p.ldb + c];
      }
      __syncthreads();
      if (has_row) {
#pragma unroll
        for (int t = 0; t < QUADS; ++t) {
          const int kk = 4 * lane + 256 * t;
#pragma unroll
          for (int c = 0; c < WP; ++c) {
            const float4 b = *reinterpret_cast<const float4*>(&Bs[c][kk]);
            acc[c] = fmaf(a[t].x, b.x, acc[c]);
            acc[c] = fmaf(a[t].y, b.y, acc[c]);
            acc[c] = fmaf(a[t].z, b.z, acc[c]);
            acc[c] = fmaf(a[t].w, b.w, acc[c]);
          }
        }
      }
    }

    // Sum over the 64 lanes (xor butterfly); lane c then holds column c.
#pragma unroll
    for (int c = 0; c < WP; ++c) {
      float v = acc[c];
      v += __shfl_xor(v, 1);
      v += __shfl_xor(v, 2);
      v += __shfl_xor(v, 4);
      v += __shfl_xor(v, 8);
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 32);
      if (has_row && lane == c && c < p.N) {
        float* cp = p.C + row * p.ldc + c;
        *cp = epilogue(v, p.alpha, p.beta, cp);
      }
    }
  }
}

// Smallest instantiated width (1, 2, 4, 8, 16) that covers n.
int padded_width(int n) {
  int w = 1;
  while (w < n) w *= 2;
  return w;
}

template <int RP, bool TA, bool TB>
hipError_t launch_rows_t(const Problem& p, hipStream_t s) {
  const int64_t nblocks = ceil_div(p.N, 16);
  const int64_t grid = nblocks < kMaxWorkItems / FewRows<RP>::THREADS
                           ? nblocks : kMaxWorkItems / FewRows<RP>::THREADS;
  hipLaunchKernelGGL((k_few_rows<RP, TA, TB>), dim3(static_cast<unsigned>(grid)),
                     dim3(FewRows<RP>::THREADS), 0, s, p, nblocks);
  return hipGetLastError();
}

template <int WP, bool TB>
hipError_t launch_cols_t(const Problem& p, hipStream_t s) {
  const int64_t nblocks = ceil_div(p.M, kRowsPerBlock);
  const int64_t grid = nblocks < kMaxWorkItems / kColThreads ? nblocks
                                                              : kMaxWorkItems / kColThreads;
  hipLaunchKernelGGL((k_few_cols<WP, TB>), dim3(static_cast<unsigned>(grid)), dim3(kColThreads), 0, s,
                     p, nblocks);
  return hipGetLastError();
}

}  // namespace

Geometry few_rows_geometry(int M, int N, int K) {
  const int rp = padded_width(M);
  const int threads = rp <= 4 ? FewRows<4>::THREADS : FewRows<16>::THREADS;
  Geometry g = make_geometry(rp, N, K, rp, 16, rp <= 4 ? FewRows<4>::KSWEEP
                                                       : FewRows<16>::KSWEEP, threads);
  return g;
}

template <bool TA, bool TB>
hipError_t launch_rows_op(const Problem& p, hipStream_t s) {
  switch (padded_width(p.M)) {
    case 1: return launch_rows_t<1, TA, TB>(p, s);
    case 2: return launch_rows_t<2, TA, TB>(p, s);
    case 4: return launch_rows_t<4, TA, TB>(p, s);
    case 8: return launch_rows_t<8, TA, TB>(p, s);
    case 16: return launch_rows_t<16, TA, TB>(p, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_few_rows(const Problem& p, hipStream_t s) {
  if (p.trans_a && p.trans_b) return launch_rows_op<true, true>(p, s);
  if (p.trans_a) return launch_rows_op<true, false>(p, s);
  if (p.trans_b) return launch_rows_op<false, true>(p, s);
  return launch_rows_op<false, false>(p, s);
}

Geometry few_cols_geometry(int M, int N, int K) {
  const int wp = padded_width(N);
  return make_geometry(M, wp, K, kRowsPerBlock, wp, wp <= 8 ? 2048 : 1024, kColThreads);
}

template <bool TB>
hipError_t launch_cols_op(const Problem& p, hipStream_t s) {
  switch (padded_width(p.N)) {
    case 1: return launch_cols_t<1, TB>(p, s);
    case 2: return launch_cols_t<2, TB>(p, s);
    case 4: return launch_cols_t<4, TB>(p, s);
    case 8: return launch_cols_t<8, TB>(p, s);
    case 16: return launch_cols_t<16, TB>(p, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_few_cols(const Problem& p, hipStream_t s) {
  if (p.trans_a) return hipErrorInvalidValue;  // the dispatcher never sends these
  return p.trans_b ? launch_cols_op<true>(p, s) : launch_cols_op<false>(p, s);
}

}  // namespace sgemm
