/*
 * sgemm.h -- C ABI of libsgemm, single-precision GEMM for MI355X (gfx950).
 *
 * Operation (all entry points that compute):
 *
 *     C := alpha * A * B + beta * C
 *
 * with A an M x K, B a K x N and C an M x N matrix of IEEE binary32 values.
 * The operation and its shapes are the ones defined in "SGEMM CUDA kernel
 * (First Half)" (introduction: S for single precision, GEMM for
 * C = alpha*A*B + beta*C, A is M x K, B is K x N, C is M x N, K the inner
 * dimension) and used by every kernel of "Optimizing Matrix Multiplication in
 * CUDA" and "1D Register Tiling: One Thread, TM Outputs" (section "The
 * Kernel": the epilogue alpha * acc + beta * C).
 *
 * Layout: row-major with leading dimensions, as in the pages' OFFSET(row, col)
 * = row * ncols + col addressing ("SGEMM CUDA kernel (First Half)", "Part 1:
 * CPU version") with the row stride made explicit:
 *     A(i, k) = A[i * lda + k],  B(k, j) = B[k * ldb + j],  C(i, j) = C[i * ldc + j].
 * Requirements: lda >= max(1, K), ldb >= max(1, N), ldc >= max(1, N), and
 * M, N, K <= 2^31 - 1025 (tile and slab coordinates then stay inside int).
 *
 * Memory and ownership: A, B and C are DEVICE pointers (e.g. from hipMalloc or
 * a torch CUDA tensor) owned by the caller.  The library allocates no device
 * memory and keeps no pointer after it returns.  C must not overlap A or B
 * (checked, error -10); A and B may overlap each other.  The check compares
 * address spans, from an operand's first addressed element to its last, so
 * sub-matrices of one allocation whose rows interleave (e.g. disjoint column
 * ranges of the same rows, sharing no element) are refused as well.
 *
 * Streams: work is enqueued on `stream` (0 = the null stream) and the call
 * returns without waiting for it; the usual stream ordering applies.  There is
 * no implicit synchronisation.  Calls are thread-safe: the only global state is
 * read-only after its first use (the dispatch table, each kernel's occupancy and
 * the device's compute-unit count, computed once), and the one piece of mutable
 * state, the variant of sgemm_last_variant, is per calling thread.  The library records no
 * memset and allocates nothing, so calls may be captured into a HIP graph.
 *
 * Semantics of the special cases:
 *   - M == 0 or N == 0: nothing is done (returns 0).
 *   - alpha == 0 or K == 0: A and B are not read; C := beta * C.
 *   - beta == 0: C is not read (NaN or Inf in C do not propagate); C := alpha * A * B.
 *   The "beta == 0 skips the read of C" reading follows "Optimizing
 *   Matrix Multiplication in CUDA", section "1D Thread Tiling", whose epilogue
 *   does not read C when beta is zero.
 *
 * Rounding: products are accumulated in fp32 with fused multiply-adds in an
 * order that depends on the kernel variant ("SGEMM CUDA kernel (First Half)",
 * "Part 4", section "FMA": one rounding per multiply-add).  Results differ from
 * an exact product only by fp32 rounding; integer-valued inputs whose partial
 * sums stay below 2^24 in magnitude give exact results.
 *
 * Transposed operands (sgemm_op, sgemm_op_ex):
 *
 *     C := alpha * op(A) * op(B) + beta * C,   op(X) = X or X^T,
 *
 * op(A) M x K, op(B) K x N.  With op(A) = A^T the stored A is K x M,
 * A^T(i, k) = A[k * lda + i], lda >= max(1, M); with op(B) = B^T the stored B
 * is N x K, B^T(k, j) = B[j * ldb + k], ldb >= max(1, K).  A row-major K x M
 * array read as its transpose is the column-major M x K matrix, so these entry
 * points also serve column-major callers.  The LDS kernels read both stored
 * forms with coalesced global loads and transpose while staging into LDS, the
 * staging transpose of "SGEMM CUDA kernel (First Half)", "Part 5: Reduced bank
 * conflict (v3)" (the A tile is written k-major into shared memory); the
 * LDS-free kernel of small grids loads either form straight into registers.
 *
 * Return codes (never aborts, never prints):
 *    0   success (work enqueued, or a valid quick return);
 *   -i   argument i is invalid (1-based, BLAS style): M=1, N=2, K=3, alpha=4,
 *        A=5, lda=6, B=7, ldb=8, beta=9, C=10, ldc=11, stream=12,
 *        variant=13 (sgemm_ex only); nothing is enqueued.  In sgemm_op and
 *        sgemm_op_ex the positions include the two leading characters:
 *        transa=1, transb=2, M=3, N=4, K=5, alpha=6, A=7, lda=8, B=9, ldb=10,
 *        beta=11, C=12, ldc=13, stream=14, variant=15 (sgemm_op_ex only);
 *   +e   a hipError_t returned by the kernel launch.
 */
#ifndef LIBSGEMM_SGEMM_H
#define LIBSGEMM_SGEMM_H

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SGEMM_API __attribute__((visibility("default")))

/* C := alpha*A*B + beta*C on `stream`, variant chosen by shape and alignment.
 * Null A or B is accepted only when alpha == 0 or K == 0; null C only when
 * M == 0 or N == 0. */
SGEMM_API int sgemm(int M, int N, int K, float alpha,
                    const float *A, int lda,
                    const float *B, int ldb,
                    float beta, float *C, int ldc,
                    hipStream_t stream);

/* As sgemm, with the kernel variant forced (0 <= variant < sgemm_num_variants()),
 * or chosen as sgemm does when variant < 0.  Returns -13 when the id is out of
 * range, names a transposed-operand variant (those serve sgemm_op_ex only), or
 * a precondition of the variant fails:
 *   - vector variants ("_vec") need A, B and C 16-byte aligned and lda, ldb,
 *     ldc, K and N multiples of 4;
 *   - variants other than "_wide" ones address one workgroup's operand panels
 *     with 32-bit offsets and need ((BM-1)*lda + BK)*4 < 2^32 and
 *     ((BK-1)*ldb + BN)*4 < 2^32 (sgemm itself switches to a "_wide" variant
 *     when these fail, so it has no such limit).
 * The operation performed is the same for every variant; only speed and fp32
 * rounding order differ.  Used by the autotuner, the bench and the tests. */
SGEMM_API int sgemm_ex(int M, int N, int K, float alpha,
                       const float *A, int lda,
                       const float *B, int ldb,
                       float beta, float *C, int ldc,
                       hipStream_t stream, int variant);

/* C := alpha*op(A)*op(B) + beta*C (see "Transposed operands" above).  transa and
 * transb are 'N' or 'n' (as stored), or 'T', 't', 'C' or 'c' (transposed; for
 * real data the conjugate transpose is the transpose); anything else returns
 * -1 or -2.  sgemm_op('N', 'N', ...) computes exactly what sgemm computes.  Null
 * pointers, overlap and quick returns follow sgemm, with the stored extents:
 * A spans (rows-1)*lda + cols elements for its stored rows x cols, B likewise. */
SGEMM_API int sgemm_op(char transa, char transb, int M, int N, int K, float alpha,
                       const float *A, int lda,
                       const float *B, int ldb,
                       float beta, float *C, int ldc,
                       hipStream_t stream);

/* As sgemm_op with the kernel variant forced, as sgemm_ex.  Returns -15 when the
 * id is out of range, when the variant's transposition (info[11], info[12]) is
 * not the requested one, or when a precondition of the variant fails: "_vec"
 * variants need A, B and C 16-byte aligned and lda, ldb, ldc, N and the stored
 * row lengths of A and B (K or M, N or K) multiples of 4; narrow variants need
 * one workgroup's stored panel spans to fit 32-bit byte offsets, as for sgemm_ex
 * with the panel's stored rows and columns. */
SGEMM_API int sgemm_op_ex(char transa, char transb, int M, int N, int K, float alpha,
                          const float *A, int lda,
                          const float *B, int ldb,
                          float beta, float *C, int ldc,
                          hipStream_t stream, int variant);

/* Number of kernel variants (ids 0 .. n-1). */
SGEMM_API int sgemm_num_variants(void);

/* Static name of a variant, e.g. "mfma32_128x128x16_w64x64_vec"; NULL when out of range. */
SGEMM_API const char *sgemm_variant_name(int variant);

/* Tile parameters of a variant, written to info[0 .. n-1] (n >= 9):
 *   info[0] kind (0 = MFMA, 1 = vector FMA), info[1] BM, info[2] BN,
 *   info[3] BK, info[4] WM (MFMA wave tile rows) or TM (VALU microtile rows),
 *   info[5] WN or TN, info[6] threads per workgroup, info[7] vector loads (0/1),
 *   info[8] LDS bytes per workgroup (0 for the LDS-free variants "mfma32r_", whose BK
 *   is the K span of the loads they keep in flight); when n >= 10, info[9] 64-bit offsets (0/1); when
 *   n >= 11, info[10] the number of k-groups splitting K inside one workgroup (1 = none);
 *   when n >= 13, info[11] and info[12]: the variant reads A, resp. B, transposed (0/1);
 *   when n >= 14, info[13]: B is loaded four consecutive k at a time and staged with k
 *   contiguous in LDS (0/1; "_bq" variants, 32-bit loads only); when n >= 15, info[14]:
 *   the number of LDS stages of a variant that loads its operands straight from global memory
 *   into LDS (0: loads go through registers; "mfma32l_" variants); when n >= 16, info[15]:
 *   the variant is persistent, launching one workgroup per resident slot that loops over
 *   output tiles ("_ps"; 0/1); when n >= 17, info[16]: the edge of the MFMA blocks, 32
 *   (v_mfma_f32_32x32x2_f32) or 16 (v_mfma_f32_16x16x4_f32, "mfma16l_" variants), 0 for
 *   the vector-FMA variants.
 *   Variants with info[11] or info[12] set serve only sgemm_op / sgemm_op_ex.
 * Returns 0, or -1 for a bad id or n < 9. */
SGEMM_API int sgemm_variant_info(int variant, int *info, int n);

/* The variant id sgemm would use for these arguments (pure host function, no GPU
 * call); -1 when the arguments describe a quick return or are invalid. */
SGEMM_API int sgemm_select_variant(int M, int N, int K,
                                   const float *A, int lda,
                                   const float *B, int ldb,
                                   const float *C, int ldc);

/* The variant id sgemm_op would use (pure host function); -1 when the arguments
 * describe a quick return or are invalid. */
SGEMM_API int sgemm_op_select_variant(char transa, char transb, int M, int N, int K,
                                      const float *A, int lda,
                                      const float *B, int ldb,
                                      const float *C, int ldc);

/* The variant id of the calling thread's most recent computing call (sgemm,
 * sgemm_ex, sgemm_op, sgemm_op_ex) when that call enqueued a GEMM kernel; -1 when
 * it enqueued none (an invalid argument, M == 0 or N == 0, the alpha == 0 / K == 0
 * scale path, a failed launch) or when this thread has made no such call.  The
 * value is kept per host thread, so concurrent callers on other threads do not
 * change it.  Pure host function. */
SGEMM_API int sgemm_last_variant(void);

/* Host-side copy of the workgroup -> output-tile map every kernel uses (for tests):
 * fills tile_m[w], tile_n[w] for w in [0, tiles_m * tiles_n).  Returns 0, or -1
 * on a bad argument. */
SGEMM_API int sgemm_tile_order(int tiles_m, int tiles_n, int group_m,
                               int *tile_m, int *tile_n);

/* Library version string. */
SGEMM_API const char *sgemm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBSGEMM_SGEMM_H */
