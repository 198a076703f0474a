/*
 * gemm_oracle.c -- the CPU oracle for dense row-major fp32 C = A x B (and
 * for the sum of an fp32 array, at the end of this file).
 *
 * TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT PATH.  Only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg may load this
 * library.  It shares no source, header or helper with the HIP library.
 *
 * What it computes.  Every page agrees on the definition: element (i, j) of
 * the product is the dot product of row i of A with column j of B
 * ("Optimizing a WebGPU Matmul Kernel using Subgroups", section 1 Naive;
 * "WebGPU 行列積の限界を測る", the N x N definition and the CPU triple loop).
 * The CPU loop on that last page keeps its running sum in a JavaScript
 * number, i.e. an IEEE binary64 value, and rounds once when it stores into a
 * Float32Array.  This oracle does the same:
 *
 *   Cd[i][j] = sum over k = 0 .. K-1, in ascending k, of (double)A[i][k] * (double)B[k][j]
 *   C[i][j]  = (float)Cd[i][j]                       (round to nearest even)
 *   ABS[i][j]= sum over k of |(double)A[i][k] * (double)B[k][j]|
 *
 * ABS is the scale of the element-wise tolerance used by the parity tests.
 *
 * Exactness facts a reader can check:
 *   - the product of two binary32 values has at most 48 significant bits, so
 *     it is exact in binary64; fused or unfused multiply-add cannot differ;
 *   - each element is summed in ascending k whatever the loop nest, so the
 *     result does not depend on the number of threads.
 *
 * Layout (readings where the pages are silent): row-major with leading
 * dimensions, A[i*lda + k], B[k*ldb + j], C[i*ldc + j], lda >= K, ldb >= N,
 * ldc >= N.  Only the M x N window of C is written.  K = 0 gives +0.0.
 *
 * Loop order is i (parallel over threads), then k, then j: row i of the
 * result is built in two binary64 row buffers while B is read row by row.
 * No blocking, no reassociation.  Build without -ffast-math.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* Status codes of this library (independent of the HIP library's). */
#define ORACLE_OK 0
#define ORACLE_BAD_ARG 1
#define ORACLE_NO_MEMORY 2

int oracle_version(void) { return 1; }

void oracle_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/*
 * oracle_gemm_f64acc
 *   M, N, K        sizes (>= 0)
 *   A, lda         M x K row-major, lda >= K
 *   B, ldb         K x N row-major, ldb >= N
 *   C, ldc         output, rounded to binary32; may be NULL
 *   Cd, ldcd       output, the binary64 sum before rounding; may be NULL
 *   ABS, ldabs     output, sum of |products| in binary64; may be NULL
 * Returns ORACLE_OK, ORACLE_BAD_ARG or ORACLE_NO_MEMORY.
 */
int oracle_gemm_f64acc(int64_t M, int64_t N, int64_t K,
                       const float *A, int64_t lda,
                       const float *B, int64_t ldb,
                       float *C, int64_t ldc,
                       double *Cd, int64_t ldcd,
                       double *ABS, int64_t ldabs) {
  if (M < 0 || N < 0 || K < 0) return ORACLE_BAD_ARG;
  if (M == 0 || N == 0) return ORACLE_OK;
  if (lda < K || ldb < N) return ORACLE_BAD_ARG;
  if (C && ldc < N) return ORACLE_BAD_ARG;
  if (Cd && ldcd < N) return ORACLE_BAD_ARG;
  if (ABS && ldabs < N) return ORACLE_BAD_ARG;
  if (K > 0 && (!A || !B)) return ORACLE_BAD_ARG;

  int failed = 0;
#pragma omp parallel
  {
    double *acc = (double *)malloc((size_t)N * sizeof(double));
    double *mag = (double *)malloc((size_t)N * sizeof(double));
    if (!acc || !mag) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t i = 0; i < M; ++i) {
      if (!acc || !mag) continue;
      for (int64_t j = 0; j < N; ++j) {
        acc[j] = 0.0;
        mag[j] = 0.0;
      }
      for (int64_t k = 0; k < K; ++k) {
        const double a = (double)A[i * lda + k];
        const float *brow = B + k * ldb;
        for (int64_t j = 0; j < N; ++j) {
          const double p = a * (double)brow[j];
          acc[j] += p;
          mag[j] += fabs(p);
        }
      }
      for (int64_t j = 0; j < N; ++j) {
        if (C) C[i * ldc + j] = (float)acc[j];
        if (Cd) Cd[i * ldcd + j] = acc[j];
        if (ABS) ABS[i * ldabs + j] = mag[j];
      }
    }
    free(acc);
    free(mag);
  }
  return failed ? ORACLE_NO_MEMORY : ORACLE_OK;
}

/*
 * oracle_gemm_elems -- the same definition evaluated at a list of (i, j)
 * positions only, for spot checks of products too large to compute whole.
 *   rows[t], cols[t]  the positions, 0 <= rows[t] < M, 0 <= cols[t] < N
 *   C, Cd, ABS        one value per position (any may be NULL)
 */
int oracle_gemm_elems(int64_t M, int64_t N, int64_t K,
                      const float *A, int64_t lda,
                      const float *B, int64_t ldb,
                      int64_t count, const int64_t *rows, const int64_t *cols,
                      float *C, double *Cd, double *ABS) {
  if (M < 0 || N < 0 || K < 0 || count < 0) return ORACLE_BAD_ARG;
  if (lda < K || ldb < N) return ORACLE_BAD_ARG;
  if (count > 0 && (!rows || !cols)) return ORACLE_BAD_ARG;
  for (int64_t t = 0; t < count; ++t)
    if (rows[t] < 0 || rows[t] >= M || cols[t] < 0 || cols[t] >= N)
      return ORACLE_BAD_ARG;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < count; ++t) {
    const int64_t i = rows[t], j = cols[t];
    double acc = 0.0, mag = 0.0;
    for (int64_t k = 0; k < K; ++k) {
      const double p = (double)A[i * lda + k] * (double)B[k * ldb + j];
      acc += p;
      mag += fabs(p);
    }
    if (C) C[t] = (float)acc;
    if (Cd) Cd[t] = acc;
    if (ABS) ABS[t] = mag;
  }
  return ORACLE_OK;
}

/*
 * oracle_gemm_ex_f64acc -- the same product with either operand stored
 * transposed, and the BLAS-style update C = alpha * op(A) op(B) + beta * C.
 *
 * Readings (the pages define only C = A x B): op(A)[i][k] is A[i*lda + k]
 * when transA is 0 and A[k*lda + i] when it is 1 (A then stored K x M, the
 * pre-transposed operand that "Optimizing a WebGPU Matmul Kernel using
 * Subgroups" section 7 uses for B); op(B)[k][j] is B[k*ldb + j] or, when
 * transB is 1, B[j*ldb + k] (B stored N x K).  alpha and beta are binary32
 * values.  When beta is 0, C's input is not read (so NaN there does not
 * propagate), as in BLAS.
 *
 *   S[i][j]  = sum over k, ascending, of op(A)[i][k] * op(B)[k][j]   (binary64, exact products)
 *   Cd[i][j] = alpha * S[i][j] + beta * Cin[i][j]                    (binary64)
 *   C[i][j]  = (float)Cd[i][j]
 *   ABS[i][j]= |alpha| * sum over k of |products| + |beta * Cin[i][j]|
 *
 *   Cin, ldcin     the input C (read only when beta != 0; may alias C)
 * Pitches: lda >= (transA ? M : K), ldb >= (transB ? K : N).
 *
 * oracle_gemm_fused_f64acc adds the rest of a fused epilogue ("fuse kernels:
 * one memory pass fewer", "GPU compute shaders", Performance): a bias row
 * vector broadcast down the columns and an elementwise activation.  Readings:
 * bias[j] is added to every row's column j (NULL: no bias); act 0 is the
 * identity and act 1 is ReLU, relu(x) = (x < 0 ? +0 : x), which keeps NaN.
 *
 *   Cd[i][j] = act(alpha * S[i][j] + beta * Cin[i][j] + bias[j])   (binary64)
 *   C[i][j]  = (float)Cd[i][j]
 *   ABS[i][j]= |alpha| * sum of |products| + |beta * Cin[i][j]| + |bias[j]|
 *
 * (ReLU commutes with the rounding to binary32, so where it is applied does
 * not change C.)  oracle_gemm_ex_f64acc is the case bias = NULL, act = 0.
 */
int oracle_gemm_fused_f64acc(int transA, int transB, int64_t M, int64_t N, int64_t K,
                             float alpha, const float *A, int64_t lda,
                             const float *B, int64_t ldb, float beta,
                             const float *Cin, int64_t ldcin,
                             const float *bias, int act,
                             float *C, int64_t ldc,
                             double *Cd, int64_t ldcd,
                             double *ABS, int64_t ldabs) {
  if (act != 0 && act != 1) return ORACLE_BAD_ARG;
  if (M < 0 || N < 0 || K < 0) return ORACLE_BAD_ARG;
  if (M == 0 || N == 0) return ORACLE_OK;
  if (lda < (transA ? M : K) || ldb < (transB ? K : N)) return ORACLE_BAD_ARG;
  if (C && ldc < N) return ORACLE_BAD_ARG;
  if (Cd && ldcd < N) return ORACLE_BAD_ARG;
  if (ABS && ldabs < N) return ORACLE_BAD_ARG;
  if (K > 0 && (!A || !B)) return ORACLE_BAD_ARG;
  if (beta != 0.0f && (!Cin || ldcin < N)) return ORACLE_BAD_ARG;

  int failed = 0;
#pragma omp parallel
  {
    double *acc = (double *)malloc((size_t)N * sizeof(double));
    double *mag = (double *)malloc((size_t)N * sizeof(double));
    if (!acc || !mag) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t i = 0; i < M; ++i) {
      if (!acc || !mag) continue;
      for (int64_t j = 0; j < N; ++j) {
        acc[j] = 0.0;
        mag[j] = 0.0;
      }
      for (int64_t k = 0; k < K; ++k) {
        const double a = (double)(transA ? A[k * lda + i] : A[i * lda + k]);
        for (int64_t j = 0; j < N; ++j) {
          const double b = (double)(transB ? B[j * ldb + k] : B[k * ldb + j]);
          const double p = a * b;
          acc[j] += p;
          mag[j] += fabs(p);
        }
      }
      for (int64_t j = 0; j < N; ++j) {
        double v = (double)alpha * acc[j];
        double m = fabs((double)alpha) * mag[j];
        if (beta != 0.0f) {
          const double c = (double)beta * (double)Cin[i * ldcin + j];
          v += c;
          m += fabs(c);
        }
        if (bias) {
          v += (double)bias[j];
          m += fabs((double)bias[j]);
        }
        if (act == 1 && v < 0.0) v = 0.0;
        if (C) C[i * ldc + j] = (float)v;
        if (Cd) Cd[i * ldcd + j] = v;
        if (ABS) ABS[i * ldabs + j] = m;
      }
    }
    free(acc);
    free(mag);
  }
  return failed ? ORACLE_NO_MEMORY : ORACLE_OK;
}

int oracle_gemm_ex_f64acc(int transA, int transB, int64_t M, int64_t N, int64_t K,
                          float alpha, const float *A, int64_t lda,
                          const float *B, int64_t ldb, float beta,
                          const float *Cin, int64_t ldcin,
                          float *C, int64_t ldc,
                          double *Cd, int64_t ldcd,
                          double *ABS, int64_t ldabs) {
  return oracle_gemm_fused_f64acc(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, Cin,
                                  ldcin, 0, 0, C, ldc, Cd, ldcd, ABS, ldabs);
}

/*
 * oracle_sum_f64acc -- the sum of n binary32 values.
 *
 * The reduction of "GPU compute shaders" (How it works: one partial sum per
 * group, then the partials combined) computes the plain sum of the array; a
 * rerun gives the same bits only when the group count and the order are
 * fixed (its Pitfalls).  Here the definition itself, written out: x[0] +
 * x[1] + ... + x[n-1] in ascending index order in binary64, rounded once to
 * binary32.  *sum_f64 is the binary64 sum before rounding, *abs_f64 the sum
 * of |x[i]| (the tolerance scale).  n = 0 gives +0.0.  Serial, so the result
 * is one fixed order.
 */
int oracle_sum_f64acc(int64_t n, const float *x, float *sum_f32, double *sum_f64,
                      double *abs_f64) {
  if (n < 0 || (n > 0 && !x) || !sum_f32) return ORACLE_BAD_ARG;
  double s = 0.0, a = 0.0;
  for (int64_t i = 0; i < n; ++i) {
    const double v = (double)x[i];
    s += v;
    a += fabs(v);
  }
  *sum_f32 = (float)s;
  if (sum_f64) *sum_f64 = s;
  if (abs_f64) *abs_f64 = a;
  return ORACLE_OK;
}
