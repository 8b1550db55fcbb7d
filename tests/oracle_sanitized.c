/*
 * Driver that runs the C oracle (oracle/gemm_oracle.c) under the address and
 * undefined-behaviour sanitizers (tests/test_host_sanitized.py; no GPU).
 * Every buffer is allocated to exactly the extent its leading dimension
 * implies -- (rows - 1) * ld + cols elements -- so a read or write past a
 * matrix, or into another thread's accumulator, is reported.  The results
 * are compared bit for bit with a literal i-j-k triple loop in fp64, which
 * sums each element in the same ascending-k order; the 16-bit product is
 * compared with the fp32 product of the same small integers.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_gemm_f32(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda,
                    const float *B, int64_t ldb, float *C, int64_t ldc);
int oracle_gemm_f32_elems(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda,
                          const float *B, int64_t ldb, int64_t count, const int64_t *ii,
                          const int64_t *jj, float *out);
int oracle_gemm_mixed(int64_t M, int64_t N, int64_t K, const uint16_t *A, int64_t lda,
                      const uint16_t *B, int64_t ldb, int format, float *C, int64_t ldc);

static int failures = 0;

static size_t extent(int64_t rows, int64_t cols, int64_t ld) {
  return rows > 0 && cols > 0 ? (size_t)((rows - 1) * ld + cols) : 1;
}

static float value(uint32_t *state) { /* small integers in [-4, 4], exact everywhere */
  *state = *state * 1664525u + 1013904223u;
  return (float)((int)(*state >> 28) % 9 - 4);
}

static void run(int64_t M, int64_t N, int64_t K, int64_t pa, int64_t pb, int64_t pc) {
  const int64_t lda = (K > 1 ? K : 1) + pa, ldb = (N > 1 ? N : 1) + pb, ldc = (N > 1 ? N : 1) + pc;
  float *A = malloc(extent(M, K, lda) * sizeof(float));
  float *B = malloc(extent(K, N, ldb) * sizeof(float));
  float *C = malloc(extent(M, N, ldc) * sizeof(float));
  uint16_t *A16 = malloc(extent(M, K, lda) * sizeof(uint16_t));
  uint16_t *B16 = malloc(extent(K, N, ldb) * sizeof(uint16_t));
  float *C16 = malloc(extent(M, N, ldc) * sizeof(float));
  uint32_t st = (uint32_t)(M * 131 + N * 17 + K);
  for (size_t i = 0; i < extent(M, K, lda); ++i) {
    A[i] = value(&st);
    uint32_t bits;
    memcpy(&bits, &A[i], 4);
    A16[i] = (uint16_t)(bits >> 16); /* bf16: small integers are exact */
  }
  for (size_t i = 0; i < extent(K, N, ldb); ++i) {
    B[i] = value(&st);
    uint32_t bits;
    memcpy(&bits, &B[i], 4);
    B16[i] = (uint16_t)(bits >> 16);
  }
  if (oracle_gemm_f32(M, N, K, A, lda, B, ldb, C, ldc) != 0 ||
      oracle_gemm_mixed(M, N, K, A16, lda, B16, ldb, 0, C16, ldc) != 0) {
    printf("FAIL rc %lldx%lldx%lld\n", (long long)M, (long long)N, (long long)K);
    ++failures;
  }
  for (int64_t i = 0; i < M; ++i)
    for (int64_t j = 0; j < N; ++j) {
      double s = 0.0;
      for (int64_t k = 0; k < K; ++k) s += (double)A[i * lda + k] * (double)B[k * ldb + j];
      if (C[i * ldc + j] != (float)s || C16[i * ldc + j] != (float)s) {
        if (failures < 10)
          printf("FAIL %lldx%lldx%lld at %lld,%lld\n", (long long)M, (long long)N, (long long)K,
                 (long long)i, (long long)j);
        ++failures;
      }
    }
  if (M > 0 && N > 0) {
    int64_t ii[3] = {0, M - 1, M / 2}, jj[3] = {N - 1, 0, N / 2};
    float out[3];
    if (oracle_gemm_f32_elems(M, N, K, A, lda, B, ldb, 3, ii, jj, out) != 0) ++failures;
    for (int t = 0; t < 3; ++t)
      if (out[t] != C[ii[t] * ldc + jj[t]]) ++failures;
  }
  free(A), free(B), free(C), free(A16), free(B16), free(C16);
}

int main(void) {
  const int64_t sizes[] = {0, 1, 2, 3, 5, 8, 17, 33};
  for (int a = 0; a < 8; ++a)
    for (int b = 0; b < 8; ++b)
      for (int c = 0; c < 8; ++c) {
        run(sizes[a], sizes[b], sizes[c], 0, 0, 0);
        if ((a + b + c) % 3 == 0) run(sizes[a], sizes[b], sizes[c], 3, 1, 5);
      }
  run(129, 67, 300, 2, 7, 1);
  printf("oracle under sanitizers: %d failures\n", failures);
  return failures == 0 ? 0 : 1;
}
