"""libsgemm: single-precision GEMM (C <- alpha*A@B + beta*C, row-major) for
the AMD Instinct MI355X (gfx950), a ladder of hand-written HIP kernels behind a
C ABI.  The binding lives in `sgemm`; importing the package loads nothing."""
