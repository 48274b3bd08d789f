/*
 * oracle_sgemm.c -- plain CPU reference for single-precision GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may load, link or
 * call this file or the library built from it: only the test suite, the
 * package's smoke check and the benchmark's CPU-baseline leg use it.  It
 * shares no code, header, table or helper with the HIP library.
 *
 * What it computes (the plain definition every kernel on the pages reaches,
 * only in a different summation order):
 *
 *     ref[i][j] = alpha * sum_{k<K} A[i][k] * B[k][j]  +  beta * C[i][j]
 *
 * for 0 <= i < M, 0 <= j < N, with A, B, C row-major and row strides lda,
 * ldb, ldc.  Sources: "SGEMM 六级优化：核心代码的演化" (daleiyang), the K1
 * kernel, whose store line is alpha*acc + beta*C over row-major A (M x K) and
 * B (K x N); CMU 11-868 lecture 4 notes (semidirectx), section 5.2, the BLAS
 * sgemm contract C = alpha*op(A)*op(B) + beta*C with op = identity here, and
 * section 5.3 for the leading dimension (mirrored to the row stride for
 * row-major storage).
 *
 * Readings where the pages are silent (BLAS conventions):
 *   - alpha == 0 or K == 0: the product is not formed and A, B are not read;
 *     ref = beta*C.
 *   - beta == 0: C is not read (a NaN in C does not propagate); ref = alpha*sum.
 *
 * Arithmetic: every float32 x float32 product is exact in float64 (24+24
 * significant bits <= 53); the sum is taken in ascending k in float64 and is
 * never rounded to float32.  Besides ref the oracle returns
 * sumabs[i][j] = sum_k |A[i][k]*B[k][j]|, the scale of the rounding error any
 * float32 evaluation of the sum can make, used by the checker's normalised
 * error.  Build with -ffp-contract=off so no fused multiply-add changes the
 * float64 rounding.
 *
 * Work split: one thread per contiguous block of rows (POSIX threads); each
 * output row is produced by exactly one thread in the same order, so results
 * do not depend on the thread count.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

typedef struct {
    int64_t row_begin, row_end;
    int64_t N, K;
    double alpha, beta;
    const float *A; int64_t lda;
    const float *B; int64_t ldb;
    const float *C; int64_t ldc;
    double *ref, *sumabs;     /* dense M x N outputs, row stride N */
    int form_product;         /* 0 when alpha == 0 or K == 0 */
} oracle_job;

static void *oracle_rows(void *arg)
{
    const oracle_job *jb = (const oracle_job *)arg;
    for (int64_t i = jb->row_begin; i < jb->row_end; ++i) {
        double *acc = jb->ref + i * jb->N;
        double *sab = jb->sumabs + i * jb->N;
        memset(acc, 0, (size_t)jb->N * sizeof(double));
        memset(sab, 0, (size_t)jb->N * sizeof(double));
        if (jb->form_product) {
            /* i-k-j order: row i of A times the rows of B, still ascending k
             * for every output element. */
            for (int64_t k = 0; k < jb->K; ++k) {
                const double a = (double)jb->A[i * jb->lda + k];
                const float *brow = jb->B + k * jb->ldb;
                for (int64_t j = 0; j < jb->N; ++j) {
                    const double p = a * (double)brow[j];
                    acc[j] += p;
                    sab[j] += fabs(p);
                }
            }
        }
        for (int64_t j = 0; j < jb->N; ++j) {
            double out = jb->form_product ? jb->alpha * acc[j] : 0.0;
            if (jb->beta != 0.0)
                out += jb->beta * (double)jb->C[i * jb->ldc + j];
            acc[j] = out;
        }
    }
    return NULL;
}

/* Threads the oracle uses when asked for 0: every core this process may run on. */
int oracle_default_threads(void)
{
#ifdef _SC_NPROCESSORS_ONLN
    long n = sysconf(_SC_NPROCESSORS_ONLN);
    return n > 0 ? (int)n : 1;
#else
    return 1;
#endif
}

/*
 * oracle_sgemm_f64: ref and sumabs are caller-allocated dense M x N float64
 * buffers (row stride N).  nthreads <= 0 means oracle_default_threads().
 * Returns the number of threads that ran (fewer than asked if a thread
 * could not be started: its rows then run on the calling thread), or a
 * negative value for invalid arguments (-1 M, -2 N, -3 K, -6 lda, -8 ldb,
 * -11 ldc, -5/-7/-10 null pointers needed for the call, -13 output
 * pointers) or -14 when the bookkeeping could not be allocated.
 */
int oracle_sgemm_f64(int64_t M, int64_t N, int64_t K, float alpha,
                     const float *A, int64_t lda, const float *B, int64_t ldb,
                     float beta, const float *C, int64_t ldc,
                     double *ref, double *sumabs, int nthreads)
{
    if (M < 0) return -1;
    if (N < 0) return -2;
    if (K < 0) return -3;
    if (lda < (K > 1 ? K : 1)) return -6;
    if (ldb < (N > 1 ? N : 1)) return -8;
    if (ldc < (N > 1 ? N : 1)) return -11;
    const int form_product = (alpha != 0.0f) && (K > 0);
    if (M > 0 && N > 0) {
        if (form_product && A == NULL) return -5;
        if (form_product && B == NULL) return -7;
        if (beta != 0.0f && C == NULL) return -10;
        if (ref == NULL || sumabs == NULL) return -13;
    }
    if (M == 0 || N == 0) return 0;

    if (nthreads <= 0) nthreads = oracle_default_threads();
    if (nthreads > M) nthreads = (int)M;
    if (nthreads < 1) nthreads = 1;

    oracle_job *jobs = (oracle_job *)calloc((size_t)nthreads, sizeof(oracle_job));
    pthread_t *tids = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !tids) { free(jobs); free(tids); return -14; }

    const int64_t per = M / nthreads, extra = M % nthreads;
    int64_t r = 0;
    for (int t = 0; t < nthreads; ++t) {
        oracle_job *jb = &jobs[t];
        jb->row_begin = r;
        r += per + (t < extra ? 1 : 0);
        jb->row_end = r;
        jb->N = N; jb->K = K;
        jb->alpha = (double)alpha; jb->beta = (double)beta;
        jb->A = A; jb->lda = lda;
        jb->B = B; jb->ldb = ldb;
        jb->C = C; jb->ldc = ldc;
        jb->ref = ref; jb->sumabs = sumabs;
        jb->form_product = form_product;
    }
    int started = 0;
    for (int t = 1; t < nthreads; ++t) {
        if (pthread_create(&tids[t], NULL, oracle_rows, &jobs[t]) != 0) {
            /* fall back to running the remaining blocks on this thread */
            for (int u = t; u < nthreads; ++u) oracle_rows(&jobs[u]);
            break;
        }
        started = t;
    }
    oracle_rows(&jobs[0]);
    for (int t = 1; t <= started; ++t) pthread_join(tids[t], NULL);
    free(jobs);
    free(tids);
    return started + 1;  /* the threads created, and this one */
}
