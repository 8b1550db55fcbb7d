/*
 * CPU oracle for C = A x B in fp32 -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load this library.  It shares no source, header or helper with the GPU
 * library; the product path never calls it.
 *
 * What it computes.  The plain definition of the product, which every tiled
 * kernel on the pages reaches again after re-associating the k sum:
 *
 *     C[i][j] = sum_{k = 0}^{K-1} A[i][k] * B[k][j]
 *
 * (page 3, ijyty.com, the naive-review paragraph: C[row][col] is the dot
 * product of row `row` of A and column `col` of B summed along K; page 4,
 * "CUDA 编程系列之三", section 6, P[row][col] = sum_k M[row][k] x N[k][col];
 * page 2, "CUDA 深入浅出（二）", first section: tiling removes no arithmetic.)
 *
 * Precision.  The pages fix only the element type (float).  Here every
 * product of two fp32 values is formed in fp64, where it is exact (24 + 24
 * significant bits <= 53), the K terms are added in fp64 in ascending k, and
 * the sum is rounded once to fp32 (round to nearest even).  That equals the
 * literal i-j-k triple loop in fp64 bit for bit, because each element still
 * sums in ascending k; only the loop nest is i-k-j so that the inner loop
 * walks a row of B.
 *
 * Layout.  Row-major with leading dimensions: A[i][k] = A[i*lda + k],
 * B[k][j] = B[k*ldb + j], C[i][j] = C[i*ldc + j].  C is overwritten, never
 * read (no alpha, beta = 0: the pages assign C, they never accumulate into it).
 *
 * No blocking, no SIMD intrinsics, no fast-math.  Rows are independent, so
 * the OpenMP split over rows is deterministic.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_BAD_ARG 1
#define ORACLE_NO_MEMORY 2

static int check_args(int64_t M, int64_t N, int64_t K, int64_t lda,
                      int64_t ldb, int64_t ldc) {
  if (M < 0 || N < 0 || K < 0) return ORACLE_BAD_ARG;
  if (lda < (K > 1 ? K : 1) || ldb < (N > 1 ? N : 1) ||
      ldc < (N > 1 ? N : 1))
    return ORACLE_BAD_ARG;
  return ORACLE_OK;
}

/* Whole product: C (M x N) = A (M x K) * B (K x N). */
int oracle_gemm_f32(int64_t M, int64_t N, int64_t K, const float *A,
                    int64_t lda, const float *B, int64_t ldb, float *C,
                    int64_t ldc) {
  int rc = check_args(M, N, K, lda, ldb, ldc);
  if (rc != ORACLE_OK) return rc;
  if (M == 0 || N == 0) return ORACLE_OK;
  int failed = 0;
#pragma omp parallel
  {
    double *acc = (double *)malloc((size_t)N * sizeof(double));
    if (acc == NULL) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(static)
    for (int64_t i = 0; i < M; ++i) {
      if (acc == NULL) continue;
      for (int64_t j = 0; j < N; ++j) acc[j] = 0.0;
      for (int64_t k = 0; k < K; ++k) {
        const double a = (double)A[i * lda + k];
        const float *brow = B + k * ldb;
        for (int64_t j = 0; j < N; ++j) acc[j] += a * (double)brow[j];
      }
      for (int64_t j = 0; j < N; ++j) C[i * ldc + j] = (float)acc[j];
    }
    free(acc);
  }
  return failed ? ORACLE_NO_MEMORY : ORACLE_OK;
}

/*
 * Selected elements only: out[t] = C[ii[t]][jj[t]] for t < count, each by the
 * same definition (fp64 sum in ascending k, one rounding to fp32).  Lets a
 * test check sampled outputs of a product too large to form on the host.
 */
int oracle_gemm_f32_elems(int64_t M, int64_t N, int64_t K, const float *A,
                          int64_t lda, const float *B, int64_t ldb,
                          int64_t count, const int64_t *ii, const int64_t *jj,
                          float *out) {
  int rc = check_args(M, N, K, lda, ldb, N > 1 ? N : 1);
  if (rc != ORACLE_OK) return rc;
  for (int64_t t = 0; t < count; ++t)
    if (ii[t] < 0 || ii[t] >= M || jj[t] < 0 || jj[t] >= N)
      return ORACLE_BAD_ARG;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < count; ++t) {
    const int64_t i = ii[t], j = jj[t];
    double s = 0.0;
    for (int64_t k = 0; k < K; ++k)
      s += (double)A[i * lda + k] * (double)B[k * ldb + j];
    out[t] = (float)s;
  }
  return ORACLE_OK;
}

/*
 * ---- 16-bit inputs, fp32 result ------------------------------------------
 *
 * The pages name the matrix-core path with FP16 / BF16 inputs as the step
 * beyond the fp32 tiled kernel (page 1, geek-doc.cn "矩阵乘法 tiling",
 * section 五: the Tensor Core row of its performance table and the closing
 * paragraph on the register / warp / instruction block pyramid).  They do
 * not spell that product out; the reading taken here is the definition
 * above over the values the 16-bit codes stand for:
 *
 *     C[i][j] = sum_k value(A[i][k]) * value(B[k][j])   (fp32 result)
 *
 * value() follows the published formats:
 *   bf16   the upper 16 bits of an IEEE 754 binary32 word (1 sign bit,
 *          8 exponent bits with bias 127, 7 fraction bits);
 *   fp16   IEEE 754 binary16 (1 sign bit, 5 exponent bits with bias 15,
 *          10 fraction bits; exponent 0 holds zero and the subnormals
 *          f * 2^-24, exponent 31 infinity and NaN).
 * Every product of two such values is exact in fp64 (at most 11 + 11
 * significant bits), the K terms are added in fp64 in ascending k and the
 * sum is rounded once to fp32, exactly as in oracle_gemm_f32.
 */
#define ORACLE_BF16 0
#define ORACLE_F16 1

static double value_bf16(uint16_t h) {
  const uint32_t w = (uint32_t)h << 16;
  float f;
  memcpy(&f, &w, sizeof f);
  return (double)f;
}

static double value_f16(uint16_t h) {
  const int sign = h >> 15, e = (h >> 10) & 0x1f, f = h & 0x3ff;
  double v;
  if (e == 0)
    v = ldexp((double)f, -24);                /* zero, subnormals */
  else if (e == 31)
    v = f ? (double)NAN : (double)INFINITY;
  else
    v = ldexp((double)(1024 + f), e - 25);    /* (1 + f/1024) * 2^(e-15) */
  return sign ? -v : v;
}

static double value16(uint16_t h, int format) {
  return format == ORACLE_BF16 ? value_bf16(h) : value_f16(h);
}

/* out[t] = value(in[t]) for t < n. */
int oracle_decode16(int64_t n, const uint16_t *in, int format, double *out) {
  if (n < 0 || (format != ORACLE_BF16 && format != ORACLE_F16)) return ORACLE_BAD_ARG;
  for (int64_t t = 0; t < n; ++t) out[t] = value16(in[t], format);
  return ORACLE_OK;
}

int oracle_gemm_mixed(int64_t M, int64_t N, int64_t K, const uint16_t *A,
                      int64_t lda, const uint16_t *B, int64_t ldb, int format,
                      float *C, int64_t ldc) {
  int rc = check_args(M, N, K, lda, ldb, ldc);
  if (rc != ORACLE_OK) return rc;
  if (format != ORACLE_BF16 && format != ORACLE_F16) return ORACLE_BAD_ARG;
  if (M == 0 || N == 0) return ORACLE_OK;
  int failed = 0;
#pragma omp parallel
  {
    double *acc = (double *)malloc((size_t)N * sizeof(double));
    if (acc == NULL) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(static)
    for (int64_t i = 0; i < M; ++i) {
      if (acc == NULL) continue;
      for (int64_t j = 0; j < N; ++j) acc[j] = 0.0;
      for (int64_t k = 0; k < K; ++k) {
        const double a = value16(A[i * lda + k], format);
        const uint16_t *brow = B + k * ldb;
        for (int64_t j = 0; j < N; ++j) acc[j] += a * value16(brow[j], format);
      }
      for (int64_t j = 0; j < N; ++j) C[i * ldc + j] = (float)acc[j];
    }
    free(acc);
  }
  return failed ? ORACLE_NO_MEMORY : ORACLE_OK;
}

/* Selected elements of the same product (see oracle_gemm_f32_elems). */
int oracle_gemm_mixed_elems(int64_t M, int64_t N, int64_t K, const uint16_t *A,
                            int64_t lda, const uint16_t *B, int64_t ldb,
                            int format, int64_t count, const int64_t *ii,
                            const int64_t *jj, float *out) {
  int rc = check_args(M, N, K, lda, ldb, N > 1 ? N : 1);
  if (rc != ORACLE_OK) return rc;
  if (format != ORACLE_BF16 && format != ORACLE_F16) return ORACLE_BAD_ARG;
  for (int64_t t = 0; t < count; ++t)
    if (ii[t] < 0 || ii[t] >= M || jj[t] < 0 || jj[t] >= N)
      return ORACLE_BAD_ARG;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < count; ++t) {
    const int64_t i = ii[t], j = jj[t];
    double s = 0.0;
    for (int64_t k = 0; k < K; ++k)
      s += value16(A[i * lda + k], format) * value16(B[k * ldb + j], format);
    out[t] = (float)s;
  }
  return ORACLE_OK;
}

/* Number of OpenMP threads a parallel region would use (for reports). */
int oracle_num_threads(void) {
  int n = 1;
#pragma omp parallel
  {
#pragma omp single
    {
#ifdef _OPENMP
      extern int omp_get_num_threads(void);
      n = omp_get_num_threads();
#endif
    }
  }
  return n;
}
