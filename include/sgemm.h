/*
 * sgemm.h -- libsgemm, single-precision GEMM on row-major matrices for the
 * AMD Instinct MI355X (gfx950).
 *
 *     C <- alpha * A * B + beta * C
 *
 * Sources this interface follows (web pages; cited by short key in the
 * library's sources):
 *   [SIX]   daleiyang.github.io, "SGEMM 六级优化：核心代码的演化"
 *           (SGEMM in six levels: how the core code evolves)
 *   [CP04]  smarter.xin, "CUDA-Practice：04 从 Shared Memory Tiling 到寄存器外积"
 *   [L04]   semidirectx.com, CMU 11-868 lecture 4 notes,
 *           "GPU 加速：分块、内存并行、稀疏矩阵与 cuBLAS"
 *   [GEMM2] pinghaoyang.com.cn, "GPU GEMM 优化完全拆解（二）：
 *           寄存器分块、向量化访存与 Warp Tiling"
 *
 * The operation is the one every kernel of [SIX] computes (the store line of
 * its K1 kernel: alpha*acc + beta*C over row-major A (M x K), B (K x N),
 * C (M x N)), with the BLAS sgemm contract of [L04] section 5.2
 * (C = alpha*op(A)*op(B) + beta*C, op = identity here) and the leading
 * dimension of [L04] section 5.3, mirrored for row-major storage: ld is the
 * number of elements between the starts of consecutive ROWS.
 *
 * Element (i, j) of A is A[i*lda + j]; of B, B[i*ldb + j]; of C, C[i*ldc + j].
 *
 * Ownership and concurrency
 *   The caller owns every buffer; A, B and C are device pointers in the
 *   HBM of the device that `stream` feeds (the current device for the null
 *   stream).  The only memory the library takes is split K's
 *   workspace (level 10 splits K for deep problems with few output tiles;
 *   hip_sgemm_plan tells beforehand whether a shape does and how many bytes
 *   it takes; hip_sgemm_tile_split says where they come from); it keeps no
 *   other state and needs no handle; calls on different streams may run
 *   concurrently.  C must not overlap A or B (undefined, unchecked, as in
 *   BLAS).
 *
 * Asynchrony
 *   Every call enqueues its kernels on `stream` (0 = the null stream) and
 *   returns without synchronising; a stream under graph capture records
 *   them, and the graph replays the call.  Argument errors are detected on
 *   the host before anything is enqueued.
 *
 * Conventions where the pages are silent (BLAS conventions)
 *   - M == 0 or N == 0: nothing is launched, returns 0.
 *   - K == 0 or alpha == 0: C <- beta*C; A and B are never read.
 *   - beta == 0: C is write-only (never read; NaN in C does not propagate).
 *   - Only the M x N window of C is written; elements of the rows' padding
 *     (columns N .. ldc-1) are never touched.
 *   - Only 4-byte (float) alignment is required, for any lda, ldb, ldc:
 *     128-bit global accesses on gfx950 need no more, so the vector paths
 *     serve every stride; partial 4-element groups at the K and N edges are
 *     loaded and stored element-wise (the page kernels of [SIX] K6 that drop
 *     the last partial float4 group are not followed).
 *   - Accumulation is float32 (round to nearest even, fused multiply-add);
 *     the summation order differs between levels.
 *
 * Status codes (return value of every compute entry point)
 *   0             success (the work is enqueued)
 *   -i (1..12)    the i-th argument of hip_sgemm is invalid, BLAS style
 *                 ("which parameter is illegal", [L04] section 5.3):
 *                 -1 M < 0, -2 N < 0, -3 K < 0, -5 A is NULL although it is
 *                 read, -6 lda < max(1, K), -7 B is NULL although it is read,
 *                 -8 ldb < max(1, N), -10 C is NULL with M, N > 0,
 *                 -11 ldc < max(1, N).  hip_sgemm_level numbers its
 *                 arguments the same way (level is not counted).
 *   -100          unknown level
 *   -101          unknown tile shape or split count (hip_sgemm_tile_split)
 *   -102, -103    op(A), op(B) not 'N' / 'T' (hip_sgemm_ex)
 *   -104          split K would need more than the fixed workspace of
 *                 hip_sgemm_ex_noalloc
 *   > 0           the hipError_t the launch reported
 */
#ifndef LIBSGEMM_SGEMM_H
#define LIBSGEMM_SGEMM_H

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SGEMM_STATUS_UNKNOWN_LEVEL (-100)
#define SGEMM_STATUS_UNKNOWN_CONFIG (-101)
#define SGEMM_STATUS_BAD_OP_A (-102)
#define SGEMM_STATUS_BAD_OP_B (-103)
#define SGEMM_STATUS_WORKSPACE_LIMIT (-104)

/*
 * Best kernel for the shape: C <- alpha*A*B + beta*C.
 * A: M x K device matrix, row stride lda >= max(1, K).
 * B: K x N device matrix, row stride ldb >= max(1, N).
 * C: M x N device matrix, row stride ldc >= max(1, N), read only if beta != 0.
 */
int hip_sgemm(int M, int N, int K, float alpha,
              const float *A, int lda,
              const float *B, int ldb,
              float beta, float *C, int ldc,
              hipStream_t stream);

/*
 * The full BLAS sgemm form: C <- alpha*op(A)*op(B) + beta*C with
 * op(X) = X or X^T ([L04] section 5.2's op(A), op(B); row-major storage as
 * everywhere in this library).
 *   op_a  'N' (or 0): A is M x K, lda >= max(1, K);
 *         'T' or 'C' (or 1): A is stored K x M and op(A) = A^T, lda >= max(1, M).
 *   op_b  'N': B is K x N, ldb >= max(1, N);
 *         'T' or 'C': B is stored N x K, op(B) = B^T, ldb >= max(1, K).
 *   (lower case accepted; for real data the conjugate transpose is the
 *   transpose.)  C is always M x N, ldc >= max(1, N), read only if beta != 0.
 * Runs level 10's plans with the operands read in place (no transposed copy
 * is made): the tile kernels stage either orientation into the same k-major
 * LDS layout.  Returns hip_sgemm's status codes (argument numbers refer to
 * hip_sgemm's positions: -6 lda, -8 ldb, ...), -102 / -103 for a bad op_a /
 * op_b.
 */
int hip_sgemm_ex(int op_a, int op_b, int M, int N, int K, float alpha,
                 const float *A, int lda,
                 const float *B, int ldb,
                 float beta, float *C, int ldc,
                 hipStream_t stream);

/*
 * hip_sgemm_ex without any device memory allocation, for the callers that
 * cannot allocate: code being captured into a HIP graph, serving loops that
 * must not call hipMalloc, harnesses that forbid allocation.  Same
 * arguments, status codes, plans and kernels as hip_sgemm_ex, and the same
 * results bit for bit.  The one plan that needs workspace, split K, takes
 * its S x M x N floats of partial sums from a fixed array in device memory
 * that the library holds on each GPU it runs on until the process ends
 * (SGEMM_NOALLOC_WORKSPACE_BYTES; every split-K plan the library chooses
 * fits it, and hip_sgemm_plan gives a shape's bytes); a call that would
 * need more returns -104 with nothing enqueued.  "A device" is the one
 * `stream` feeds (the current device for the null stream), whichever device
 * is current on the calling thread.  The first call on a device looks the
 * array's address up (making that device current for the lookup and then
 * restoring the caller's); no call allocates or frees.
 * The array is shared by every call on one GPU and keeps the last call's
 * contents (a call reads back only what it has written): calls that overlap
 * in time on one GPU (other streams, other host threads) race on it, and
 * their results are undefined.  Serialise them.
 */
#define SGEMM_NOALLOC_WORKSPACE_BYTES (8LL << 20)

int hip_sgemm_ex_noalloc(int op_a, int op_b, int M, int N, int K, float alpha,
                         const float *A, int lda,
                         const float *B, int ldb,
                         float beta, float *C, int ldc,
                         hipStream_t stream);

/*
 * Same operation with the rung of the optimisation ladder forced.  Every
 * level is correct for every shape and alignment.  Levels (the page kernels
 * each one re-designs for gfx950):
 *   0 naive, consecutive lanes walk consecutive ROWS ([SIX] K1)
 *   1 naive, consecutive lanes walk consecutive COLUMNS ([SIX] K2;
 *     [L04] section 1.1)
 *   2 LDS tiles 32 x 32, one output per thread, two barriers per phase,
 *     padded rows ([SIX] K3; [CP04] tiled_gemm; [L04] sections 2.2-2.5)
 *   3 thread coarsening, 4 column tiles per block ([SIX] K3c; [CP04]
 *     coarse_gemm; [L04] section 2.7)
 *   4 1-D register tile, 8 rows per thread ([SIX] K4; [GEMM2] kernel 4)
 *   5 2-D register tile, 128 x 128 block, 8 x 8 outer product per thread
 *     ([SIX] K5; [CP04] register_tiling_gemm; [GEMM2] kernel 5)
 *   6 128-bit loads, A transposed in LDS, 128-bit LDS reads ([SIX] K6;
 *     [GEMM2] kernel 6)
 *   7 double-buffered LDS, one barrier per K step ([CP04]
 *     double_buffer_gemm)
 *   8 wave tiling (block -> 64 x 64 wave tiles -> lane sub-tiles) ([GEMM2]
 *     warp tiling section; its thread-swizzling block order measured slower
 *     on this rung on MI355X, so tiles go in plain order)
 *   9 FP32 matrix cores (v_mfma_f32_32x32x2_f32 and v_mfma_f32_16x16x4_f32)
 *     on the level-8 pipeline
 *  10 shape-aware dispatch, the level hip_sgemm runs (hip_sgemm_plan names
 *     the plan a shape gets): M <= 16 or N <= 16 on the thin kernels
 *     (vector-ALU FMA chains for one to four rows or columns, otherwise
 *     one 16-row matrix-core block; cross-lane sums in a fixed order);
 *     fewer than 128 tiles of 64 x 64 on the thin matrix-core kernel over
 *     16-row panels; a deep K over a small grid, or K >= 2048 over a wide,
 *     shallow one, split over K into workspace planes that a second
 *     kernel adds in order; otherwise one of three whole-tile kernels
 *     whose K loop is hand-scheduled assembly (256 x 128, 128 x 128, and
 *     64 x 64 over four K-slice wavefronts), with partial edge tiles, or
 *     with whole tiles plus a fringe: one row and / or one column is
 *     summed by the tiles' own blocks in the same launch (each fringe
 *     output by one block, its per-k partial sums added in k order; grids
 *     of at least 4 x 8 tiles of 256 x 128, 8 x 8 of 128 x 128, 16 x 16
 *     of 64 x 64), up to 16 beside the two large tiles by the thin
 *     kernels.  A call enqueues up to
 *     three kernels on the stream, over disjoint parts of C ([GEMM2]
 *     size-sweep section: a library is many kernels picked by shape)
 */
int hip_sgemm_level(int level, int M, int N, int K, float alpha,
                    const float *A, int lda,
                    const float *B, int ldb,
                    float beta, float *C, int ldc,
                    hipStream_t stream);

/*
 * Level 9's matrix-core kernel with its configuration forced, for tuning
 * sweeps (the per-shape choices of level 10 were measured with it):
 *   tile    0 .. hip_sgemm_num_tiles()-1: 256 x 128 (BK 16, 8 wavefronts),
 *           128 x 128 (BK 32, 4), 128 x 64 (BK 16, 4), 64 x 64 (BK 16, 4),
 *           and with each stage cut into two K slices whose sums meet in LDS
 *           (twice the wavefronts): 128 x 128 (BK 32, 8), 64 x 64 (BK 32, 8);
 *           6: level 10's 64 x 64 assembly-loop tile (BK 64 split over four
 *           wavefronts; where it does not fit, tile 5 stands in);
 *           7 ..: a catalogue of further legal configurations of level 9's
 *           tile template (block tile, stage depth, wavefront grid, matrix
 *           block size, K slices), row-major operands, for sweeps over the
 *           template's parameter space ([GEMM2] autotuning section: the
 *           best parameters differ per GPU and are searched);
 *           hip_sgemm_tile_name gives each one's parameters;
 *   splits  >= 1: the K range is cut into about `splits` slices (each a
 *           multiple of the tile's BK; ceil(K / slice) of them run) that
 *           compute separately, and a second kernel adds the slices' float32
 *           sums in slice order, then applies alpha and beta ([GEMM2]
 *           size-sweep section: split-K, a tiled GEMM plus a reduce kernel).
 *           splits = 1, or a slice covering all of K, is the unsplit kernel
 *           (for tiles 0 and 1 on whole tiles, level 10's version of them
 *           with the K loop in assembly; for tile 0 the same results bit
 *           for bit when K % 16 == 0).
 * Split K needs S x M x N floats of workspace: the library takes it from a
 * stream-ordered memory pool of its own (one per device -- the device that
 * `stream` feeds --, created on first use, memory kept cached until the
 * process ends), allocated and released on `stream` around the two kernels;
 * concurrent calls never share it.  On a
 * stream under graph capture it is a stream-ordered allocation from the
 * device's default pool instead (recorded as a graph memory node).  Results
 * are bit-reproducible for a given (tile, splits, shape).  Other arguments,
 * quick returns and status codes as hip_sgemm; -101 for a bad tile or
 * splits < 1.
 */
int hip_sgemm_tile_split(int tile, int splits, int M, int N, int K, float alpha,
                         const float *A, int lda,
                         const float *B, int ldb,
                         float beta, float *C, int ldc,
                         hipStream_t stream);

/* Number of tile shapes hip_sgemm_tile_split accepts, and their names
 * ("256x128x16_8w", ..., "cat_64x64x32_1x1w_m16", ...: block tile x stage
 * depth first; NULL if unknown; static, owned by the library). */
int hip_sgemm_num_tiles(void);
const char *hip_sgemm_tile_name(int tile);

/* Number of levels (valid levels are 0 .. hip_sgemm_num_levels()-1). */
int hip_sgemm_num_levels(void);

/* Short name of a level ("L9_mfma_f32", ...); NULL if unknown.  The
 * string is static and owned by the library. */
const char *hip_sgemm_level_name(int level);

/* Human-readable text for a status code; static, owned by the library. */
const char *hip_sgemm_status_string(int status);

/*
 * The level hip_sgemm picks for a shape and alignment (the same rule it
 * applies), without launching anything.  Returns the level, or a negative
 * status for invalid sizes.
 */
int hip_sgemm_auto_level(int M, int N, int K,
                         const float *A, int lda,
                         const float *B, int ldb,
                         const float *C, int ldc);

/*
 * Launch geometry a level would use for a shape, without launching: the
 * number of workgroups, threads per workgroup, K steps each workgroup walks
 * (ceil(K / BK): the boundary rule of [L04] section 2.5 rounds the phase
 * count up and zero-fills the tail), and the output tile (tile_m x tile_n)
 * each workgroup owns.  For level 10 this is its largest launch (the tile
 * grid, or the thin kernel).  Any output pointer may be NULL.  Returns 0, or
 * a negative status.
 */
int hip_sgemm_launch_shape(int level, int M, int N, int K,
                           long long *workgroups, int *threads_per_group,
                           long long *k_steps, int *tile_m, int *tile_n);

/*
 * The plan hip_sgemm and hip_sgemm_ex take for a shape (with alpha != 0;
 * alpha == 0 is the SCALE plan whatever K), decided on the host from M, N, K
 * alone, without launching anything:
 *   *plan             one of the SGEMM_PLAN_* ids below;
 *   *launches         kernels one call enqueues on its stream (for
 *                     SGEMM_PLAN_TILES_FRINGE as hip_sgemm takes the shape
 *                     with packed operands, lda = K and ldb = N for
 *                     row-major storage: leading dimensions large enough to
 *                     put an offset at or past 2^31 bytes move a one-row /
 *                     one-column fringe to the thin kernels, one launch
 *                     per side);
 *   *workspace_bytes  device memory the call takes for split K's partial
 *                     sums (splits x M x N floats; 0 for every other plan):
 *                     the only plan that allocates.  hip_sgemm and
 *                     hip_sgemm_ex take it from the library's stream-ordered
 *                     pool (see hip_sgemm_tile_split).
 * [GEMM2] (size-sweep section) describes a library as many kernels chosen by
 * problem size, split K among them; this reports which one a shape gets.
 * Any output pointer may be NULL.  Returns 0, or -1 / -2 / -3 for a negative
 * M / N / K.
 */
#define SGEMM_PLAN_NONE 0         /* M == 0 or N == 0: nothing is launched */
#define SGEMM_PLAN_SCALE 1        /* K == 0 (or alpha == 0): C <- beta*C */
#define SGEMM_PLAN_FEW_ROWS 2     /* M <= 16: thin kernel over rows of C */
#define SGEMM_PLAN_FEW_COLS 3     /* N <= 16: thin kernel over columns of C */
#define SGEMM_PLAN_TILES 4        /* one grid of matrix-core tiles */
#define SGEMM_PLAN_TILES_FRINGE 5 /* whole tiles + a <= 16-wide fringe (see level 10) */
#define SGEMM_PLAN_SPLIT_K 6      /* tiles over K slices + an in-order reduction */
#define SGEMM_PLAN_THIN_PANELS 7  /* small problems: 16-row panels of C */

int hip_sgemm_plan(int M, int N, int K, int *plan, int *launches,
                   long long *workspace_bytes);

#ifdef __cplusplus
}
#endif

#endif /* LIBSGEMM_SGEMM_H */
