// sgemm_api.hip -- the C-ABI host layer of libsgemm: argument validation,
// BLAS quick returns, level dispatch and introspection.
//
// Validation follows the BLAS sgemm habit of reporting which parameter is
// illegal ([L04] section 5.3: a leading dimension smaller than the row length
// is an argument error).  Everything here runs on the host before any HIP
// call, so argument errors never enqueue work.
#include "../../include/sgemm.h"
#include "l9_catalogue.h"
#include "sgemm_internal.h"

namespace sgemm {
namespace {

constexpr int kNumLevels = 11;

const LevelDesc* level_desc(int level) {
  static const LevelDesc* const table[kNumLevels] = {
      level0(), level1(), level2(), level3(), level4(),
      level5(), level6(), level7(), level8(), level9(), level10(),
  };
  return table[level];
}

int max1(int v) { return v > 1 ? v : 1; }

// Returns 0 or the negative 1-based position (in hip_sgemm's argument list)
// of the first bad argument.  A stored transposed is K x M (lda >= M), B
// stored transposed is N x K (ldb >= K).
int validate(int M, int N, int K, float alpha, const void* A, int lda,
             const void* B, int ldb, const void* C, int ldc, bool ta = false,
             bool tb = false) {
  if (M < 0) return -1;
  if (N < 0) return -2;
  if (K < 0) return -3;
  if (lda < max1(ta ? M : K)) return -6;
  if (ldb < max1(tb ? K : N)) return -8;
  if (ldc < max1(N)) return -11;
  const bool product = M > 0 && N > 0 && K > 0 && alpha != 0.0f;
  if (product && A == nullptr) return -5;
  if (product && B == nullptr) return -7;
  if (M > 0 && N > 0 && C == nullptr) return -10;
  return 0;
}

int status_of(hipError_t e) { return e == hipSuccess ? 0 : static_cast<int>(e); }

// C <- beta*C; beta == 0 stores zeros without reading C.
__global__ __launch_bounds__(256) void k_scale(int M, int N, float beta,
                                               float* __restrict__ C,
                                               int64_t ldc, int64_t tiles_n,
                                               int64_t ntiles) {
  for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
    const int64_t row = (t / tiles_n) * 4 + threadIdx.x / 64;
    const int64_t col = (t % tiles_n) * 64 + threadIdx.x % 64;
    if (row < M && col < N) {
      float* c = C + row * ldc + col;
      *c = beta == 0.0f ? 0.0f : beta * *c;
    }
  }
}

int run(const LevelDesc* lv, int M, int N, int K, float alpha, const float* A,
        int lda, const float* B, int ldb, float beta, float* C, int ldc,
        hipStream_t stream) {
  const int bad = validate(M, N, K, alpha, A, lda, B, ldb, C, ldc);
  if (bad) return bad;
  if (M == 0 || N == 0) return 0;
  Problem p{M, N, K, alpha, beta, A, lda, B, ldb, C, ldc};
  if (K == 0 || alpha == 0.0f) return status_of(launch_scale(p, stream));
  return status_of(lv->launch(p, stream));
}

// hip_sgemm_tile_split's tiles: seven named shapes, then the catalogue.
constexpr int kNumTiles = 7;
constexpr int kNumTileIds = kNumTiles + SGEMM_CATALOGUE_SIZE;

const CatalogueEntry* catalogue_entry(int i) {
  int first = 0, second = 0;
  const CatalogueEntry* a = catalogue_first(&first);
  const CatalogueEntry* b = catalogue_second(&second);
  return i < first ? &a[i] : &b[i - first];
}

Shape tile_shape(int tile) {
  static const Shape shapes[kNumTiles] = {Shape::kHuge,        Shape::kLarge,      Shape::kMid,
                                          Shape::kSmall,       Shape::kLargeSliced, Shape::kSmallSliced,
                                          Shape::kSmallDeep};
  return shapes[tile];
}

int choose_level(int M, int N, int K) {
  (void)M;
  (void)N;
  (void)K;
  return 10;  // the shape-aware rung picks kernels per problem itself
}

}  // namespace

hipError_t launch_scale(const Problem& p, hipStream_t stream) {
  const Geometry g = make_geometry(p.M, p.N, 1, 4, 64, 1, 256);
  const int64_t tiles_n = ceil_div(p.N, 64);
  hipLaunchKernelGGL(k_scale, dim3(static_cast<unsigned>(g.workgroups)),
                     dim3(256), 0, stream, p.M, p.N, p.beta, p.C, p.ldc,
                     tiles_n, g.tiles);
  return hipGetLastError();
}

}  // namespace sgemm

using namespace sgemm;

extern "C" {

int hip_sgemm(int M, int N, int K, float alpha, const float* A, int lda,
              const float* B, int ldb, float beta, float* C, int ldc,
              hipStream_t stream) {
  const int bad = validate(M, N, K, alpha, A, lda, B, ldb, C, ldc);
  if (bad) return bad;
  return run(level_desc(choose_level(M, N, K)), M, N, K, alpha, A, lda, B, ldb,
             beta, C, ldc, stream);
}

int hip_sgemm_level(int level, int M, int N, int K, float alpha,
                    const float* A, int lda, const float* B, int ldb,
                    float beta, float* C, int ldc, hipStream_t stream) {
  if (level < 0 || level >= kNumLevels) return SGEMM_STATUS_UNKNOWN_LEVEL;
  return run(level_desc(level), M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
             stream);
}

int hip_sgemm_tile_split(int tile, int splits, int M, int N, int K, float alpha,
                        const float* A, int lda, const float* B, int ldb, float beta,
                        float* C, int ldc, hipStream_t stream) {
  if (tile < 0 || tile >= kNumTileIds || splits < 1) return SGEMM_STATUS_UNKNOWN_CONFIG;
  const int bad = validate(M, N, K, alpha, A, lda, B, ldb, C, ldc);
  if (bad) return bad;
  if (M == 0 || N == 0) return 0;
  Problem p{M, N, K, alpha, beta, A, lda, B, ldb, C, ldc};
  if (K == 0 || alpha == 0.0f) return status_of(launch_scale(p, stream));
  if (tile >= kNumTiles) {
    const CatalogueEntry* c = catalogue_entry(tile - kNumTiles);
    const int64_t k_split = k_split_for(K, splits, c->bk);
    if (k_split >= K) return status_of(c->launch(p, stream));
    return status_of(launch_splitk_fn(c->split, k_split, p, stream));
  }
  const Shape shape = tile_shape(tile);
  const int64_t k_split = k_split_for(K, splits, shape_bk(shape));
  if (k_split >= K) return status_of(launch_tiles(shape, p, stream));
  return status_of(launch_splitk(shape, k_split, p, stream));
}

int hip_sgemm_num_tiles(void) { return kNumTileIds; }

// 'N' / 'n' / 0: as stored; 'T' / 't' / 'C' / 'c' / 1: transposed (for real
// data the conjugate transpose is the transpose); -1 otherwise.
static int parse_op(int op) {
  switch (op) {
    case 0: case 'N': case 'n': return 0;
    case 1: case 'T': case 't': case 'C': case 'c': return 1;
    default: return -1;
  }
}

int hip_sgemm_ex(int op_a, int op_b, int M, int N, int K, float alpha, const float* A,
                 int lda, const float* B, int ldb, float beta, float* C, int ldc,
                 hipStream_t stream) {
  const int ta = parse_op(op_a), tb = parse_op(op_b);
  if (ta < 0) return SGEMM_STATUS_BAD_OP_A;
  if (tb < 0) return SGEMM_STATUS_BAD_OP_B;
  const int bad = validate(M, N, K, alpha, A, lda, B, ldb, C, ldc, ta, tb);
  if (bad) return bad;
  if (M == 0 || N == 0) return 0;
  Problem p{M, N, K, alpha, beta, A, lda, B, ldb, C, ldc};
  p.trans_a = ta != 0;
  p.trans_b = tb != 0;
  if (K == 0 || alpha == 0.0f) return status_of(launch_scale(p, stream));
  return status_of(level_desc(10)->launch(p, stream));
}

int hip_sgemm_ex_noalloc(int op_a, int op_b, int M, int N, int K, float alpha, const float* A,
                         int lda, const float* B, int ldb, float beta, float* C, int ldc,
                         hipStream_t stream) {
  const int ta = parse_op(op_a), tb = parse_op(op_b);
  if (ta < 0) return SGEMM_STATUS_BAD_OP_A;
  if (tb < 0) return SGEMM_STATUS_BAD_OP_B;
  const int bad = validate(M, N, K, alpha, A, lda, B, ldb, C, ldc, ta, tb);
  if (bad) return bad;
  if (M == 0 || N == 0) return 0;
  Problem p{M, N, K, alpha, beta, A, lda, B, ldb, C, ldc};
  p.trans_a = ta != 0;
  p.trans_b = tb != 0;
  if (K == 0 || alpha == 0.0f) return status_of(launch_scale(p, stream));
  if (plan10(M, N, K).workspace_bytes > static_workspace_bytes())
    return SGEMM_STATUS_WORKSPACE_LIMIT;
  return status_of(launch10_with(p, stream, Workspace::kStatic));
}

const char* hip_sgemm_tile_name(int tile) {
  if (tile < 0 || tile >= kNumTileIds) return nullptr;
  if (tile >= kNumTiles) return catalogue_entry(tile - kNumTiles)->name;
  static const char* const names[kNumTiles] = {"256x128x16_8w", "128x128x32_4w", "128x64x16_4w",
                                               "64x64x16_4w", "128x128x32_8w_2slices",
                                               "64x64x32_8w_2slices", "64x64x64_4w_4slices"};
  return names[tile];
}

int hip_sgemm_num_levels(void) { return kNumLevels; }

const char* hip_sgemm_level_name(int level) {
  if (level < 0 || level >= kNumLevels) return nullptr;
  return level_desc(level)->name;
}

const char* hip_sgemm_status_string(int status) {
  switch (status) {
    case 0: return "success";
    case -1: return "argument 1 (M) is negative";
    case -2: return "argument 2 (N) is negative";
    case -3: return "argument 3 (K) is negative";
    case -5: return "argument 5 (A) is NULL but A is read";
    case -6: return "argument 6 (lda) is smaller than max(1, K) (max(1, M) for a transposed A)";
    case -7: return "argument 7 (B) is NULL but B is read";
    case -8: return "argument 8 (ldb) is smaller than max(1, N) (max(1, K) for a transposed B)";
    case -10: return "argument 10 (C) is NULL with M, N > 0";
    case -11: return "argument 11 (ldc) is smaller than max(1, N)";
    case SGEMM_STATUS_UNKNOWN_LEVEL: return "unknown level";
    case SGEMM_STATUS_UNKNOWN_CONFIG: return "unknown tile shape or split count";
    case SGEMM_STATUS_BAD_OP_A: return "op(A) is not 'N' or 'T'";
    case SGEMM_STATUS_BAD_OP_B: return "op(B) is not 'N' or 'T'";
    case SGEMM_STATUS_WORKSPACE_LIMIT:
      return "split K needs more workspace than the fixed array of hip_sgemm_ex_noalloc";
    default: break;
  }
  if (status > 0) return hipGetErrorString(static_cast<hipError_t>(status));
  return "unknown status";
}

int hip_sgemm_auto_level(int M, int N, int K, const float* A, int lda,
                         const float* B, int ldb, const float* C, int ldc) {
  const int bad = validate(M, N, K, 1.0f, A, lda, B, ldb, C, ldc);
  if (bad) return bad;
  return choose_level(M, N, K);
}

int hip_sgemm_launch_shape(int level, int M, int N, int K,
                           long long* workgroups, int* threads_per_group,
                           long long* k_steps, int* tile_m, int* tile_n) {
  if (level < 0 || level >= kNumLevels) return SGEMM_STATUS_UNKNOWN_LEVEL;
  if (M < 0) return -1;
  if (N < 0) return -2;
  if (K < 0) return -3;
  const Geometry g = level_desc(level)->geometry(M, N, K);
  if (workgroups) *workgroups = g.workgroups;
  if (threads_per_group) *threads_per_group = g.threads;
  if (k_steps) *k_steps = g.k_steps;
  if (tile_m) *tile_m = g.tile_m;
  if (tile_n) *tile_n = g.tile_n;
  return 0;
}

int hip_sgemm_plan(int M, int N, int K, int* plan, int* launches, long long* workspace_bytes) {
  if (M < 0) return -1;
  if (N < 0) return -2;
  if (K < 0) return -3;
  const PlanInfo info = plan10(M, N, K);
  if (plan) *plan = info.plan;
  if (launches) *launches = info.launches;
  if (workspace_bytes) *workspace_bytes = info.workspace_bytes;
  return 0;
}

}  // extern "C"
