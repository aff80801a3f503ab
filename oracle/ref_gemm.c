/*
 * oracle/ref_gemm.c -- TEST INFRASTRUCTURE, not part of the product path.
 *
 * A plain, slow, obviously correct CPU reference for what the pipelined GEMMs
 * (fp32, and bfloat16 / binary16 inputs), the pipelined tile copy and the
 * pipelined attention compute. Only the test suite, the smoke
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
#include <stdlib.h>
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

/* Thread count of the parallel loops (timing only: results do not depend on
   it, each output element being one thread's sequential sum). */
void oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
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

/* ---- 16-bit inputs (bfloat16 / IEEE binary16), fp64 accumulation ---------
 * The BF16/FP16 form of the same product: A and B hold 16-bit values, the
 * product and the sum are taken in fp64 as above (every product of two
 * 16-bit values is exact in fp64), and C is fp64. Formats: fmt 1 = bfloat16
 * (sign, 8-bit exponent, 7-bit fraction: the upper half of a binary32),
 * fmt 2 = IEEE 754 binary16 (sign, 5-bit exponent bias 15, 10-bit fraction,
 * subnormals, infinities, NaN). */

double oracle_decode16(uint16_t h, int fmt)
{
    if (fmt == 1) {
        union { uint32_t u; float f; } v;
        v.u = (uint32_t)h << 16;
        return (double)v.f;
    } else {
        const int sign = (h >> 15) & 1;
        const int e = (h >> 10) & 0x1f;
        const int f = h & 0x3ff;
        double x;
        if (e == 0)
            x = ldexp((double)f, -24);                 /* subnormal: f * 2^-14 * 2^-10 */
        else if (e == 31)
            x = f ? NAN : INFINITY;
        else
            x = ldexp((double)(f | 0x400), e - 25);    /* (1024 + f) * 2^(e - 15 - 10) */
        return sign ? -x : x;
    }
}

/* C[i*ldc + j] = sum_{p<K} dec(A[i*lda + p]) * dec(B[p*ldb + j]) in fp64,
 * loop order i, p, j; `absolute` != 0 sums |a| * |b| instead. */
void oracle_gemm16_f64(int64_t M, int64_t N, int64_t K,
                       const uint16_t *A, int64_t lda,
                       const uint16_t *B, int64_t ldb,
                       double *C, int64_t ldc, int fmt, int absolute)
{
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < M; ++i) {
        double *c = C + i * ldc;
        int64_t j, p;
        for (j = 0; j < N; ++j)
            c[j] = 0.0;
        for (p = 0; p < K; ++p) {
            double a = oracle_decode16(A[i * lda + p], fmt);
            const uint16_t *b = B + p * ldb;
            if (absolute)
                a = fabs(a);
            for (j = 0; j < N; ++j) {
                const double bv = oracle_decode16(b[j], fmt);
                c[j] += a * (absolute ? fabs(bv) : bv);
            }
        }
    }
}

/* ---- scaled dot-product attention over 16-bit Q, K, V --------------------
 * The async copy article ("from cp.async to memcpy_async"), section 6.2,
 * "FlashAttention's tile pipeline":
 * Q tiles stay put while K/V tiles stream past them, each step scoring the
 * current K tile, rescaling the running result and accumulating V. That
 * online form reaches, up to rounding, the plain definition written here:
 *   s_j   = scale * sum_{d<D} q_d * k_jd                        (j < Sk)
 *   w_j   = exp(s_j - max_t s_t) / sum_u exp(s_u - max_t s_t)
 *   O_c   = sum_j w_j * v_jc                                    (c < Dv)
 * per query row q (i < Sq), all in fp64 from the decoded 16-bit inputs
 * (subtracting the row maximum changes nothing mathematically; it keeps
 * exp in range). Three magnitudes scale the acceptance bound:
 * Wabs_c = sum_j w_j * |v_jc|, G = max_j sum_d |q_d| * |k_jd| (the size of
 * the score sums, which fp32 accumulation perturbs) and, once per call,
 * Vmax_c = max_j |v_jc| (the size of what an underflowing weight can drop).
 * Row-major Q (Sq x D, ldq), K (Sk x D, ldk), V (Sk x Dv, ldv), O and Wabs
 * (Sq x Dv, ldo), G (Sq), Vmax (Dv); Sk >= 1; Wabs, G and Vmax may be NULL.
 * Returns 0, or -1 if scratch memory cannot be allocated. */
int oracle_attention_f64(int64_t Sq, int64_t Sk, int64_t D, int64_t Dv,
                         const uint16_t *Q, int64_t ldq, const uint16_t *K, int64_t ldk,
                         const uint16_t *V, int64_t ldv, double scale, int fmt,
                         double *O, double *Wabs, int64_t ldo, double *G, double *Vmax)
{
    int failed = 0;
    int64_t i;
    if (Vmax) {
        int64_t j, c;
        for (c = 0; c < Dv; ++c) {
            Vmax[c] = 0.0;
            for (j = 0; j < Sk; ++j) {
                const double v = fabs(oracle_decode16(V[j * ldv + c], fmt));
                if (v > Vmax[c])
                    Vmax[c] = v;
            }
        }
    }
#pragma omp parallel for schedule(static) reduction(| : failed)
    for (i = 0; i < Sq; ++i) {
        double *s = (double *)malloc((size_t)(Sk > 0 ? Sk : 1) * sizeof(double));
        double *q = (double *)malloc((size_t)(D > 0 ? D : 1) * sizeof(double));
        int64_t j, d, c;
        double mx = -INFINITY, sum = 0.0, gmax = 0.0;
        if (!s || !q) {
            free(s);
            free(q);
            failed = 1;
            continue;
        }
        for (d = 0; d < D; ++d)
            q[d] = oracle_decode16(Q[i * ldq + d], fmt);
        for (j = 0; j < Sk; ++j) {
            double acc = 0.0, mag = 0.0;
            for (d = 0; d < D; ++d) {
                const double k = oracle_decode16(K[j * ldk + d], fmt);
                acc += q[d] * k;
                mag += fabs(q[d]) * fabs(k);
            }
            s[j] = scale * acc;
            if (s[j] > mx)
                mx = s[j];
            if (mag > gmax)
                gmax = mag;
        }
        if (G)
            G[i] = gmax;
        for (j = 0; j < Sk; ++j) {
            s[j] = exp(s[j] - mx);
            sum += s[j];
        }
        for (c = 0; c < Dv; ++c) {
            O[i * ldo + c] = 0.0;
            if (Wabs)
                Wabs[i * ldo + c] = 0.0;
        }
        for (j = 0; j < Sk; ++j) {
            const double w = s[j] / sum;
            for (c = 0; c < Dv; ++c) {
                const double v = oracle_decode16(V[j * ldv + c], fmt);
                O[i * ldo + c] += w * v;
                if (Wabs)
                    Wabs[i * ldo + c] += w * fabs(v);
            }
        }
        free(s);
        free(q);
    }
    return failed ? -1 : 0;
}
