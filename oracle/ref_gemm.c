/*
 * oracle/ref_gemm.c -- TEST INFRASTRUCTURE, not part of the product path.
 *
 * A plain, slow, obviously correct CPU reference for what the pipelined FP32
 * GEMM and the pipelined tile copy compute. Only the test suite, the smoke
 * check and the CPU-baseline leg of the benchmark load this library. It shares
 * no source, header, table or helper with the HIP library; the two meet only
 * through the seeded inputs of the datagen package.
 *
 * Sources (the pages, by title and section):
 *  - "Day 74 -- Async copies and pipelines", section "Two kernels, one
 *    arithmetic": C = A*B for row-major A and B; the pipelined and the
 *    synchronous kernel compute the same product.
 *  - "pipelined_gemm.cu", function matmulCpu: the CPU reference walks rows,
 *    then the inner dimension p, then columns, accumulating in double.
 *  - "cp.async" (TVM TIRx tile-op reference), section "Example: four 16-byte
 *    copies per thread": a copy through shared memory must return the input
 *    bytes unchanged.
 *
 * Arithmetic: every product of two fp32 values is exact in fp64 (24+24 <= 53
 * significand bits); each sum is rounded once in fp64, k ascending. The error
 * of C_ref is at most K * 2^-53 * (|A||B|)_ij, negligible against the fp32
 * acceptance bound 4 * K * 2^-24 * (|A||B|)_ij.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -shared -fPIC. OpenMP splits the
 * row loop only, so every element keeps its k-ascending order and the result
 * does not depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* C[i*ldc + j] = sum_{p<K} A[i*lda + p] * B[p*ldb + j] for i<M, j<N (fp64).
 * Row-major operands with leading dimensions lda >= K, ldb >= N, ldc >= N.
 * K == 0 gives the empty sum, +0.0. Loop order i, p, j as in matmulCpu. */
void oracle_gemm_f64(int64_t M, int64_t N, int64_t K,
                     const float *A, int64_t lda,
                     const float *B, int64_t ldb,
                     double *C, int64_t ldc)
{
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < M; ++i) {
        double *c = C + i * ldc;
        int64_t j, p;
        for (j = 0; j < N; ++j)
            c[j] = 0.0;
        for (p = 0; p < K; ++p) {
            const double a = (double)A[i * lda + p];
            const float *b = B + p * ldb;
            for (j = 0; j < N; ++j)
                c[j] += a * (double)b[j];
        }
    }
}

/* Abs[i*ldc + j] = sum_{p<K} |A[i*lda + p]| * |B[p*ldb + j]| (fp64): the
 * magnitude that scales the elementwise rounding bound of an fp32 dot
 * product of length K. Same loop order and layout rules as oracle_gemm_f64. */
void oracle_abs_gemm_f64(int64_t M, int64_t N, int64_t K,
                         const float *A, int64_t lda,
                         const float *B, int64_t ldb,
                         double *Abs, int64_t ldc)
{
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < M; ++i) {
        double *c = Abs + i * ldc;
        int64_t j, p;
        for (j = 0; j < N; ++j)
            c[j] = 0.0;
        for (p = 0; p < K; ++p) {
            const double a = fabs((double)A[i * lda + p]);
            const float *b = B + p * ldb;
            for (j = 0; j < N; ++j)
                c[j] += a * fabs((double)b[j]);
        }
    }
}

/* dst[r*ldd + c] = src[r*lds + c] for r<rows, c<cols: the tile copy's result
 * is its input. Padding columns of dst (c >= cols) are not touched. */
void oracle_copy_f32(int64_t rows, int64_t cols, const float *src, int64_t lds,
                     float *dst, int64_t ldd)
{
    int64_t r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < rows; ++r)
        memcpy(dst + r * ldd, src + r * lds, (size_t)cols * sizeof(float));
}

/* Number of threads the parallel loops above use. */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
