/*
 * sgemm_ref.c -- float64 CPU oracle for single-precision GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the correctness oracle: only the
 * test-suite, the smoke check and the bench's CPU-baseline leg may load it.
 * It shares no code, header, table or helper with the HIP library.
 *
 * What it computes (the plain definition, written out):
 *
 *     C_out[i][j] = alpha * sum_{k=0}^{K-1} A[i][k] * B[k][j]  +  beta * C_in[i][j]
 *
 * with A (M x K), B (K x N) and C (M x N) row-major fp32 matrices.  Sources:
 *   - "SGEMM CUDA kernel (First Half)" (twicy.github.io), introduction: GEMM is
 *     C = alpha*A*B + beta*C, A is M x K, B is K x N, C is M x N, K the inner
 *     dimension; section "Part 1: CPU version": each output element is the dot
 *     product of one row of A and one column of B, with the OFFSET(row, col)
 *     = row * ncols + col row-major addressing.
 *   - "Optimizing Matrix Multiplication in CUDA" (mathidot), section "Baseline
 *     CPU Implementation": the same i-j-k loop nest.
 *   - "1D Register Tiling: One Thread, TM Outputs" (maxxfuu), section "The
 *     Kernel": the epilogue alpha * acc + beta * C.
 *
 * Readings taken where the pages are silent:
 *   - Accumulation is in float64, not in the pages' float: every product of two
 *     fp32 values is exact in double (24 + 24 <= 53 significand bits), and the
 *     k-order is ascending and fixed, so the result does not depend on the
 *     thread count.
 *   - Leading dimensions: element (i, k) of A sits at A[i*lda + k]; likewise
 *     B[k*ldb + j] and C[i*ldc + j].  The pages use packed matrices (ld equal to
 *     the row length); a padded ld is the same addressing with a larger stride.
 *   - beta == 0: C_in is never read (BLAS semantics; "Optimizing Matrix
 *     Multiplication in CUDA", section on 1D thread tiling, skips the read of C
 *     when beta is zero).  NaN or Inf in C_in therefore does not propagate.
 *   - alpha == 0 or K == 0: A and B are never read and C_out = beta * C_in.
 *
 * Error bound returned next to each reference value:
 *
 *     bound[i][j] = 1e-5 * (|alpha| * sum_k |A[i][k] * B[k][j]| + |beta * C_in[i][j]|) + 1e-6
 *
 * A GPU result g passes when |g - ref| <= bound element by element.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fPIC -shared (no fast-math, no
 * reassociation).
 */
#include <math.h>
#include <stddef.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_REL_TOL 1e-5
#define ORACLE_ABS_TOL 1e-6

/* One output element: reference value and its error bound. */
static void ref_element(int i, int j, int K, double alpha,
                        const float *A, long lda, const float *B, long ldb,
                        double beta, const float *C, long ldc,
                        double *ref_out, double *bound_out)
{
    double s = 0.0;   /* sum_k a_ik * b_kj, ascending k */
    double sa = 0.0;  /* sum_k |a_ik * b_kj|            */
    if (alpha != 0.0) {
        for (int k = 0; k < K; ++k) {
            double p = (double)A[(long)i * lda + k] * (double)B[(long)k * ldb + j];
            s += p;
            sa += fabs(p);
        }
    }
    double c = 0.0;
    if (beta != 0.0)
        c = beta * (double)C[(long)i * ldc + j];
    *ref_out = alpha * s + c;
    *bound_out = ORACLE_REL_TOL * (fabs(alpha) * sa + fabs(c)) + ORACLE_ABS_TOL;
}

/*
 * Reference for the rows [row_begin, row_end) of C_out.
 * ref and bound are packed row-major (row_end - row_begin) x N arrays of double.
 * C may be NULL when beta == 0; A and B may be NULL when alpha == 0 or K == 0.
 * nthreads <= 0 means "OpenMP default".  Returns 0, or -1 on a bad argument.
 */
int sgemm_ref_rows(int M, int N, int K, double alpha,
                   const float *A, long lda, const float *B, long ldb,
                   double beta, const float *C, long ldc,
                   int row_begin, int row_end,
                   double *ref, double *bound, int nthreads)
{
    if (M < 0 || N < 0 || K < 0 || row_begin < 0 || row_end > M || row_begin > row_end)
        return -1;
    if (K == 0)
        alpha = 0.0;  /* an empty sum: the alpha term is exactly zero */
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel for schedule(static)
    for (int i = row_begin; i < row_end; ++i) {
        for (int j = 0; j < N; ++j) {
            long o = (long)(i - row_begin) * N + j;
            ref_element(i, j, K, alpha, A, lda, B, ldb, beta, C, ldc, &ref[o], &bound[o]);
        }
    }
    return 0;
}

/*
 * Reference for npts individual elements (I[p], J[p]).  ref and bound have
 * npts entries.  Same conventions as sgemm_ref_rows.
 */
int sgemm_ref_points(int M, int N, int K, double alpha,
                     const float *A, long lda, const float *B, long ldb,
                     double beta, const float *C, long ldc,
                     const long *I, const long *J, long npts,
                     double *ref, double *bound, int nthreads)
{
    if (M < 0 || N < 0 || K < 0 || npts < 0)
        return -1;
    for (long p = 0; p < npts; ++p)
        if (I[p] < 0 || I[p] >= M || J[p] < 0 || J[p] >= N)
            return -1;
    if (K == 0)
        alpha = 0.0;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel for schedule(static)
    for (long p = 0; p < npts; ++p)
        ref_element((int)I[p], (int)J[p], K, alpha, A, lda, B, ldb, beta, C, ldc, &ref[p], &bound[p]);
    return 0;
}

/* Number of threads an OpenMP parallel region would use (for reporting). */
int sgemm_ref_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
