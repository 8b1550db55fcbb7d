/*
 * gemm_mixed.h -- C ABI of the 16-bit-input product of the gemm_f32 library
 * (MI355X, gfx950).
 *
 * The operation is the pages' product C = A x B, with A and B given as
 * 16-bit floating-point codes and C accumulated and returned in fp32: the
 * matrix-core step the pages put after the fp32 tiled kernel, fed FP16 or
 * BF16 inputs (geek-doc.cn "矩阵乘法 tiling", section 五: the Tensor Core
 * row of its performance table and the paragraph after it).
 *
 *   C[i][j] = sum_{k<K} value(A[i][k]) * value(B[k][j])
 *
 * value() reads a code by its published format: bf16 is the upper half of
 * an IEEE 754 binary32 word; fp16 is IEEE 754 binary16.  Every product of
 * two such values is exact in fp32; the sum is accumulated in fp32 in an
 * order the kernel chooses (integer-valued inputs whose partial sums stay
 * below 2^24 give the exact result).
 *
 * Layout (row-major, leading dimensions in elements):
 *   A[i][k] = A[i*lda + k]  16-bit codes, M x K, lda >= max(1, K)
 *   B[k][j] = B[k*ldb + j]  16-bit codes, K x N, ldb >= max(1, N)
 *   C[i][j] = C[i*ldc + j]  float, M x N, ldc >= max(1, N)
 * A and B must be 2-byte aligned and C 4-byte aligned; any leading
 * dimension is served by the same 128-bit loads (gfx950 runs with
 * unaligned global access enabled).  Only edge tiles and the last partial
 * k step use element-wise loads.
 * Elements of C outside the M x N window are never written.
 *
 * Memory, streams and errors are as for gemm_f32 (gemm_f32.h): device
 * pointers owned by the caller, nothing allocated, asynchronous on `stream`
 * (hipStream_t as void*, NULL = null stream), argument errors returned
 * before anything is enqueued, status codes GEMM_F32_*.
 */
#ifndef GEMM_MIXED_H
#define GEMM_MIXED_H

#ifdef __cplusplus
extern "C" {
#endif

/* Input formats. */
#define GEMM_MIXED_BF16 0
#define GEMM_MIXED_F16 1

/*
 * gemm_mixed -- C = A x B (overwrite) with 16-bit inputs and fp32 result.
 *   M, N, K   each >= 0.  M == 0 or N == 0: no-op.  K == 0: C is set to 0.
 *   A, B      16-bit codes in `format`; may be NULL when they hold no element.
 *   format    GEMM_MIXED_BF16 or GEMM_MIXED_F16 (else GEMM_F32_BAD_ARG).
 *   config    -1 picks a launch-table entry for the shape, otherwise an
 *             index below gemm_mixed_num_configs() (else GEMM_F32_BAD_CONFIG).
 * Returns GEMM_F32_OK or an error code of gemm_f32.h; on error nothing is
 * launched.  Kernels: entries 0-2 use BM x BN workgroup tiles with k step
 * 64, both operands staged in LDS as rows of 64 k values (B transposed on
 * the way in), two LDS stages, v_mfma_f32_32x32x16_bf16 / _f16 on 32 x 32
 * blocks per wave; entry 3 loads both operands straight into LDS in their
 * row-major layouts (16-byte aligned rows of A and B, N % 8 == 0 and K a
 * multiple of 64; otherwise it runs entry 0), reads B's operands with the
 * transposing LDS read and computes on v_mfma_f32_16x16x32_bf16 / _f16;
 * entry 4 is the same pipeline on v_mfma_f32_32x32x16_bf16 / _f16 (same
 * conditions, same fallback) and gives entry 0's bits.  The automatic
 * choice takes entry 4 for K == 64 and entry 3 for other multiples of 64
 * when 256 x 256 tiles fill the GPU.
 */
int gemm_mixed(int M, int N, int K, const void *A, int lda, const void *B,
               int ldb, float *C, int ldc, int format, int config,
               void *stream);

/* Number of launch-table entries of gemm_mixed. */
int gemm_mixed_num_configs(void);

/*
 * gemm_mixed_tile -- the entry gemm_mixed would use (host only): workgroup
 * tile BM x BN, k step BK, threads per workgroup and the entry index.  Any
 * output pointer may be NULL.  Returns GEMM_F32_OK, GEMM_F32_BAD_CONFIG or
 * GEMM_F32_INVALID_DIM.
 */
int gemm_mixed_tile(int config, int M, int N, int K, int *BM, int *BN, int *BK,
                    int *threads, int *chosen_config);

#ifdef __cplusplus
}
#endif

#endif /* GEMM_MIXED_H */
