/*
 * sgemm_blocked.c -- cache-blocked, multi-threaded CPU SGEMM: a second CPU baseline for the
 * bench, next to the plain float64 oracle.  Measurement only: the GPU library never calls it
 * and no test takes its values as expected results.
 *
 * Computes C := alpha * A * B + beta * C for row-major fp32 matrices with leading dimensions
 * (A M x K, B K x N, C M x N), the operation of "SGEMM CUDA kernel (First Half)"
 * (introduction).  Why a blocked loop: "Shared Memory and Register Blocking" (CUDA Handbook,
 * ch. 17) contrasts a cache-blocked CPU product with a plain loop to show how much a plain loop
 * understates the CPU; this is that blocked form, written here as the usual five-loop nest:
 *
 *   for jc (NC columns of B and C)
 *     for pc (KC of K):  pack B[pc:pc+KC, jc:jc+NC] into NR-wide strips (shared, parallel)
 *       for ic (MC rows, one block per thread at a time):  pack A[ic:ic+MC, pc:pc+KC] into
 *                                                           MR-tall strips (per thread)
 *         for jr, ir:  an MR x NR register tile, fp32 multiply-adds over the KC slice
 *
 * Conventions: beta == 0 never reads C; alpha == 0 or K == 0 gives beta * C without reading
 * A or B (those of the library).  Accumulation is fp32 in KC slices, so results differ from
 * an exact product by fp32 rounding only.
 */
#include <immintrin.h>
#include <omp.h>
#include <stdlib.h>
#include <string.h>

enum { MR = 6, NR = 32, MC = 96, KC = 256, NC = 3072 };

/* MR x NR tile: acc = sum over kc of Ap (packed MR-tall strip) times Bp (packed NR-wide strip). */
static void tile_generic(int kc, const float* restrict Ap, const float* restrict Bp, float* restrict acc) {
    float c[MR][NR];
    memset(c, 0, sizeof c);
    for (int k = 0; k < kc; ++k) {
        const float* b = Bp + (size_t)k * NR;
        for (int i = 0; i < MR; ++i) {
            const float a = Ap[(size_t)k * MR + i];
            for (int j = 0; j < NR; ++j) c[i][j] += a * b[j];
        }
    }
    memcpy(acc, c, sizeof c);
}

/* AVX-512: 6 rows x 2 vectors of 16 = 12 independent accumulators (enough to cover the FMA
 * latency on two FMA ports). */
__attribute__((target("avx512f"))) static void tile_avx512(int kc, const float* restrict Ap,
                                                            const float* restrict Bp, float* restrict acc) {
    __m512 c[MR][2];
    for (int i = 0; i < MR; ++i) c[i][0] = c[i][1] = _mm512_setzero_ps();
    for (int k = 0; k < kc; ++k) {
        const __m512 b0 = _mm512_loadu_ps(Bp + (size_t)k * NR);
        const __m512 b1 = _mm512_loadu_ps(Bp + (size_t)k * NR + 16);
        const float* a = Ap + (size_t)k * MR;
        for (int i = 0; i < MR; ++i) {
            const __m512 ai = _mm512_set1_ps(a[i]);
            c[i][0] = _mm512_fmadd_ps(ai, b0, c[i][0]);
            c[i][1] = _mm512_fmadd_ps(ai, b1, c[i][1]);
        }
    }
    for (int i = 0; i < MR; ++i) {
        _mm512_storeu_ps(acc + i * NR, c[i][0]);
        _mm512_storeu_ps(acc + i * NR + 16, c[i][1]);
    }
}

/* AVX2: the 6 x 32 tile as two 6 x 16 halves (12 accumulators each; 16 registers in all). */
__attribute__((target("avx2,fma"))) static void tile_avx2(int kc, const float* restrict Ap,
                                                          const float* restrict Bp, float* restrict acc) {
    for (int half = 0; half < 2; ++half) {
        __m256 c[MR][2];
        for (int i = 0; i < MR; ++i) c[i][0] = c[i][1] = _mm256_setzero_ps();
        for (int k = 0; k < kc; ++k) {
            const __m256 b0 = _mm256_loadu_ps(Bp + (size_t)k * NR + half * 16);
            const __m256 b1 = _mm256_loadu_ps(Bp + (size_t)k * NR + half * 16 + 8);
            const float* a = Ap + (size_t)k * MR;
            for (int i = 0; i < MR; ++i) {
                const __m256 ai = _mm256_broadcast_ss(a + i);
                c[i][0] = _mm256_fmadd_ps(ai, b0, c[i][0]);
                c[i][1] = _mm256_fmadd_ps(ai, b1, c[i][1]);
            }
        }
        for (int i = 0; i < MR; ++i) {
            _mm256_storeu_ps(acc + i * NR + half * 16, c[i][0]);
            _mm256_storeu_ps(acc + i * NR + half * 16 + 8, c[i][1]);
        }
    }
}

typedef void (*tile_fn)(int, const float*, const float*, float*);

static tile_fn pick_tile(void) {
    __builtin_cpu_init();
    if (__builtin_cpu_supports("avx512f")) return tile_avx512;
    if (__builtin_cpu_supports("avx2") && __builtin_cpu_supports("fma")) return tile_avx2;
    return tile_generic;
}

/* Which tile routine runs here: 2 = AVX-512, 1 = AVX2+FMA, 0 = portable C. */
int sgemm_blocked_isa(void) {
    tile_fn f = pick_tile();
    return f == tile_avx512 ? 2 : (f == tile_avx2 ? 1 : 0);
}

/* Pack B[pc:pc+kc, jc+jr*NR : ...] strip r into NR-wide rows (zero past nc). */
static void pack_b_strip(int kc, int nc, int r, const float* B, long ldb, float* dst) {
    const int j0 = r * NR;
    const int w = nc - j0 < NR ? nc - j0 : NR;
    for (int k = 0; k < kc; ++k) {
        const float* src = B + (size_t)k * ldb + j0;
        float* d = dst + (size_t)k * NR;
        int j = 0;
        for (; j < w; ++j) d[j] = src[j];
        for (; j < NR; ++j) d[j] = 0.f;
    }
}

/* Pack A[ic:ic+mc, pc:pc+kc] into MR-tall strips, k-major within a strip (zero past mc). */
static void pack_a_block(int mc, int kc, const float* A, long lda, float* dst) {
    for (int i0 = 0; i0 < mc; i0 += MR) {
        const int h = mc - i0 < MR ? mc - i0 : MR;
        float* d = dst + (size_t)i0 * kc;
        for (int k = 0; k < kc; ++k) {
            int i = 0;
            for (; i < h; ++i) d[(size_t)k * MR + i] = A[(size_t)(i0 + i) * lda + k];
            for (; i < MR; ++i) d[(size_t)k * MR + i] = 0.f;
        }
    }
}

static void scale_c(int M, int N, float beta, float* C, long ldc, int nthreads) {
#pragma omp parallel for num_threads(nthreads) schedule(static)
    for (int i = 0; i < M; ++i) {
        float* c = C + (size_t)i * ldc;
        if (beta == 0.f)
            for (int j = 0; j < N; ++j) c[j] = 0.f;
        else if (beta != 1.f)
            for (int j = 0; j < N; ++j) c[j] *= beta;
    }
}

/* Returns 0, or -1 on a bad argument or a failed allocation.  nthreads <= 0: all OpenMP threads. */
int sgemm_blocked(int M, int N, int K, float alpha, const float* A, int lda, const float* B, int ldb, float beta,
                  float* C, int ldc, int nthreads) {
    if (M < 0 || N < 0 || K < 0 || lda < (K > 1 ? K : 1) || ldb < (N > 1 ? N : 1) || ldc < (N > 1 ? N : 1))
        return -1;
    if (M == 0 || N == 0) return 0;
    if (nthreads <= 0) nthreads = omp_get_max_threads();
    scale_c(M, N, beta, C, ldc, nthreads);
    if (alpha == 0.f || K == 0) return 0;
    const tile_fn tile = pick_tile();
    float* bpack = (float*)aligned_alloc(64, sizeof(float) * (size_t)KC * NC);
    float* apack = (float*)aligned_alloc(64, sizeof(float) * (size_t)MC * KC * nthreads);
    if (!bpack || !apack) {
        free(bpack);
        free(apack);
        return -1;
    }
    for (int jc = 0; jc < N; jc += NC) {
        const int nc = N - jc < NC ? N - jc : NC;
        const int nstrips = (nc + NR - 1) / NR;
        for (int pc = 0; pc < K; pc += KC) {
            const int kc = K - pc < KC ? K - pc : KC;
#pragma omp parallel num_threads(nthreads)
            {
#pragma omp for schedule(static)
                for (int r = 0; r < nstrips; ++r)
                    pack_b_strip(kc, nc, r, B + (size_t)pc * ldb + jc, ldb, bpack + (size_t)r * kc * NR);
                float* ap = apack + (size_t)omp_get_thread_num() * MC * KC;
                float acc[MR * NR];
#pragma omp for schedule(dynamic)
                for (int ic = 0; ic < M; ic += MC) {
                    const int mc = M - ic < MC ? M - ic : MC;
                    pack_a_block(mc, kc, A + (size_t)ic * lda + pc, lda, ap);
                    for (int r = 0; r < nstrips; ++r) {
                        const int j0 = r * NR;
                        const int w = nc - j0 < NR ? nc - j0 : NR;
                        for (int i0 = 0; i0 < mc; i0 += MR) {
                            const int h = mc - i0 < MR ? mc - i0 : MR;
                            tile(kc, ap + (size_t)i0 * kc, bpack + (size_t)r * kc * NR, acc);
                            for (int i = 0; i < h; ++i) {
                                float* c = C + (size_t)(ic + i0 + i) * ldc + jc + j0;
                                for (int j = 0; j < w; ++j) c[j] += alpha * acc[i * NR + j];
                            }
                        }
                    }
                }
            }
        }
    }
    free(bpack);
    free(apack);
    return 0;
}
