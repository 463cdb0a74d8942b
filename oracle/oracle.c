/*
 * CPU oracle for the dense matrix multiply C = alpha*A*B + beta*C and for the
 * half-precision product with a fused bias + GELU(tanh) epilogue.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the GPU library links, includes or
 * calls this file; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg load it.  It shares no header, helper or constant with the
 * HIP code.
 *
 * What it computes, and where the pages define it:
 *
 *  - "SGEMM优化，从naive到warptiling", section 问题与估算 (problem statement):
 *    C = alpha * A x B + beta * C with A of M x K, B of K x N and C of M x N,
 *    all row-major single-precision floats.  The same page's naive kernel
 *    (section k1) applies it element by element as alpha*sum + beta*C.
 *  - Lecture 24 "CUDA GEMM 分块（Tiling）与 Tensor Core 思维", its opening
 *    triple-loop definition of the product: every output element is the sum
 *    over k of A[i][k] * B[k][j].
 *  - The half-precision variant (binary16 or bfloat16 inputs) with bias and activation fused into the
 *    write-back is the one described on the DeepGEMM page (sections 1.1 and
 *    3.2: bias, scaling and GELU done in registers before one store).  Its
 *    activation is read as the tanh form of GELU (Hendrycks & Gimpel 2016):
 *    gelu(x) = 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))).
 *
 * Precision: every product and sum is taken in IEEE double, with no FMA
 * contraction (built with -ffp-contract=off), summing k in ascending order for
 * each output element.  The result is returned in double, not rounded to the
 * output type.  Alongside each result the oracle returns the scale
 *     den = |alpha| * sum_k |A_ik| |B_kj| + |beta| |C_ij|
 * (for the half path: |alpha| * sum_k |a||b| + |bias_j|), the quantity that
 * bounds the rounding error of any summation order (Higham, "Accuracy and
 * Stability of Numerical Algorithms", the dot-product error bound).
 *
 * Conventions the pages leave open (plain BLAS reading):
 *  - beta == 0: C is not read, so NaN or Inf in C does not propagate.
 *  - alpha == 0 or K == 0: A and B are not read; the result is beta*C.
 *  - leading dimensions lda >= K, ldb >= N, ldc >= N; element (i,j) of A is
 *    A[i*lda + j].
 *
 * Loop structure: for each row i the oracle keeps a row of N double
 * accumulators and walks k = 0..K-1, adding A[i][k]*B[k][j] into accumulator
 * j.  Every accumulator therefore sees its K terms in ascending k, exactly the
 * per-element sum of the definition; the loop order only changes which
 * element is updated next, never the operations applied to any one element.
 * Rows are independent and split over OpenMP threads.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------- */
/* IEEE binary16 -> double, written from the format's definition:           */
/* 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits; exponent 0 holds  */
/* subnormals (fraction * 2^-24), exponent 31 holds Inf (fraction 0) or NaN.  */
/* ------------------------------------------------------------------------- */
double oracle_half_to_double(uint16_t h) {
  int sign = (h >> 15) & 1;
  int expo = (h >> 10) & 0x1f;
  int frac = h & 0x3ff;
  double v;
  if (expo == 0) {
    v = ldexp((double)frac, -24);
  } else if (expo == 31) {
    v = frac ? NAN : INFINITY;
  } else {
    v = ldexp((double)(frac + 1024), expo - 25);
  }
  return sign ? -v : v;
}

/* bfloat16 -> double: a bfloat16 value is the upper 16 bits of an IEEE binary32,
 * so it is widened by appending 16 zero bits and converted exactly. */
double oracle_bf16_to_double(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* The tanh form of GELU, evaluated in double with the C library's tanh. */
double oracle_gelu_tanh(double x) {
  const double c = sqrt(2.0 / M_PI);
  double inner = c * (x + 0.044715 * x * x * x);
  return 0.5 * x * (1.0 + tanh(inner));
}

static int oracle_threads(int requested) {
#ifdef _OPENMP
  return requested > 0 ? requested : omp_get_max_threads();
#else
  (void)requested;
  return 1;
#endif
}

/*
 * Full single-precision product.
 *   ref[i*N + j] = alpha * sum_k A[i*lda+k] * B[k*ldb+j] + beta * C0[i*ldc+j]
 *   den[i*N + j] = |alpha| * sum_k |A_ik||B_kj| + |beta| |C0_ij|   (den may be NULL)
 * ref and den are packed M x N row-major double arrays owned by the caller.
 * C0 may be NULL when beta == 0.  threads <= 0 uses the OpenMP default.
 */
void oracle_sgemm(int M, int N, int K, double alpha, const float *A, int lda,
                  const float *B, int ldb, double beta, const float *C0,
                  int ldc, double *ref, double *den, int threads) {
  int nt = oracle_threads(threads);
  int skip_product = (alpha == 0.0) || (K == 0);
#pragma omp parallel num_threads(nt)
  {
    double *acc = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
    double *mag = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
#pragma omp for schedule(dynamic, 1)
    for (int i = 0; i < M; ++i) {
      for (int j = 0; j < N; ++j) {
        acc[j] = 0.0;
        mag[j] = 0.0;
      }
      if (!skip_product) {
        for (int k = 0; k < K; ++k) {
          double a = (double)A[(size_t)i * lda + k];
          const float *brow = B + (size_t)k * ldb;
          for (int j = 0; j < N; ++j) acc[j] += a * (double)brow[j];
          if (den) {
            double aa = fabs(a);
            for (int j = 0; j < N; ++j) mag[j] += aa * fabs((double)brow[j]);
          }
        }
      }
      for (int j = 0; j < N; ++j) {
        double r = skip_product ? 0.0 : alpha * acc[j];
        double cterm = 0.0, cmag = 0.0;
        if (beta != 0.0) {
          double c = (double)C0[(size_t)i * ldc + j];
          cterm = beta * c;
          cmag = fabs(beta) * fabs(c);
        }
        ref[(size_t)i * N + j] = r + cterm;
        if (den) den[(size_t)i * N + j] = (skip_product ? 0.0 : fabs(alpha) * mag[j]) + cmag;
      }
    }
    free(acc);
    free(mag);
  }
}

/*
 * The same definition evaluated for a list of single entries (rows[t], cols[t]),
 * t < count, each as its own ascending-k dot product.  Used where the full
 * product is too large for the CPU (sampled parity at full problem size).
 */
void oracle_sgemm_entries(int K, double alpha, const float *A, int lda,
                          const float *B, int ldb, double beta, const float *C0,
                          int ldc, const int64_t *rows, const int64_t *cols,
                          int64_t count, double *ref, double *den, int threads) {
  int nt = oracle_threads(threads);
  int skip_product = (alpha == 0.0) || (K == 0);
#pragma omp parallel for num_threads(nt) schedule(static)
  for (int64_t t = 0; t < count; ++t) {
    int64_t i = rows[t], j = cols[t];
    double s = 0.0, m = 0.0;
    if (!skip_product) {
      for (int k = 0; k < K; ++k) {
        double a = (double)A[i * lda + k];
        double b = (double)B[(int64_t)k * ldb + j];
        s += a * b;
        m += fabs(a) * fabs(b);
      }
    }
    double r = skip_product ? 0.0 : alpha * s;
    double cterm = 0.0, cmag = 0.0;
    if (beta != 0.0) {
      double c = (double)C0[i * ldc + j];
      cterm = beta * c;
      cmag = fabs(beta) * fabs(c);
    }
    ref[t] = r + cterm;
    if (den) den[t] = (skip_product ? 0.0 : fabs(alpha) * m) + cmag;
  }
}

typedef double (*decode16_fn)(uint16_t);

/*
 * 16-bit inputs (binary16 or bfloat16 bit patterns, decoded exactly to double),
 * product summed in double:
 *   x = alpha * sum_k a_ik b_kj + bias[j]      (bias may be NULL: 0)
 *   ref = act(x), act 0 = identity, act 1 = GELU(tanh)
 *   den = |alpha| sum_k |a||b| + |bias[j]|
 * alpha == 0 or K == 0 leaves only bias.
 */
static void half_gemm(decode16_fn dec, int M, int N, int K, double alpha, const uint16_t *A,
                      int lda, const uint16_t *B, int ldb, const float *bias, int act,
                      double *ref, double *den, int threads) {
  int nt = oracle_threads(threads);
  int skip_product = (alpha == 0.0) || (K == 0);
  /* B decoded to double once (the conversion is exact, so this changes no value;
   * it only avoids decoding every element of B once per output row). */
  double *bdec = NULL;
  if (!skip_product && N > 0) {
    bdec = (double *)malloc(sizeof(double) * (size_t)K * (size_t)N);
#pragma omp parallel for num_threads(nt) schedule(static)
    for (int k = 0; k < K; ++k)
      for (int j = 0; j < N; ++j) bdec[(size_t)k * N + j] = dec(B[(size_t)k * ldb + j]);
  }
#pragma omp parallel num_threads(nt)
  {
    double *acc = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
    double *mag = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
#pragma omp for schedule(dynamic, 1)
    for (int i = 0; i < M; ++i) {
      for (int j = 0; j < N; ++j) {
        acc[j] = 0.0;
        mag[j] = 0.0;
      }
      if (!skip_product) {
        for (int k = 0; k < K; ++k) {
          double a = dec(A[(size_t)i * lda + k]);
          const double *brow = bdec + (size_t)k * N;
          for (int j = 0; j < N; ++j) acc[j] += a * brow[j];
          if (den) {
            double aa = fabs(a);
            for (int j = 0; j < N; ++j) mag[j] += aa * fabs(brow[j]);
          }
        }
      }
      for (int j = 0; j < N; ++j) {
        double b = bias ? (double)bias[j] : 0.0;
        double x = (skip_product ? 0.0 : alpha * acc[j]) + b;
        ref[(size_t)i * N + j] = act == 1 ? oracle_gelu_tanh(x) : x;
        if (den) den[(size_t)i * N + j] = (skip_product ? 0.0 : fabs(alpha) * mag[j]) + fabs(b);
      }
    }
    free(acc);
    free(mag);
  }
  free(bdec);
}

/* Sampled entries of the 16-bit product, one ascending-k dot product each. */
static void half_entries(decode16_fn dec, int K, double alpha, const uint16_t *A, int lda,
                         const uint16_t *B, int ldb, const float *bias, int act,
                         const int64_t *rows, const int64_t *cols, int64_t count, double *ref,
                         double *den, int threads) {
  int nt = oracle_threads(threads);
  int skip_product = (alpha == 0.0) || (K == 0);
#pragma omp parallel for num_threads(nt) schedule(static)
  for (int64_t t = 0; t < count; ++t) {
    int64_t i = rows[t], j = cols[t];
    double s = 0.0, m = 0.0;
    if (!skip_product) {
      for (int k = 0; k < K; ++k) {
        double a = dec(A[i * lda + k]);
        double b = dec(B[(int64_t)k * ldb + j]);
        s += a * b;
        m += fabs(a) * fabs(b);
      }
    }
    double bb = bias ? (double)bias[j] : 0.0;
    double x = (skip_product ? 0.0 : alpha * s) + bb;
    ref[t] = act == 1 ? oracle_gelu_tanh(x) : x;
    if (den) den[t] = (skip_product ? 0.0 : fabs(alpha) * m) + fabs(bb);
  }
}

/* binary16 inputs */
void oracle_hgemm_bias_act(int M, int N, int K, double alpha, const uint16_t *A, int lda,
                           const uint16_t *B, int ldb, const float *bias, int act, double *ref,
                           double *den, int threads) {
  half_gemm(oracle_half_to_double, M, N, K, alpha, A, lda, B, ldb, bias, act, ref, den, threads);
}

void oracle_hgemm_entries(int K, double alpha, const uint16_t *A, int lda, const uint16_t *B,
                          int ldb, const float *bias, int act, const int64_t *rows,
                          const int64_t *cols, int64_t count, double *ref, double *den,
                          int threads) {
  half_entries(oracle_half_to_double, K, alpha, A, lda, B, ldb, bias, act, rows, cols, count, ref,
               den, threads);
}

/* bfloat16 inputs */
void oracle_bgemm_bias_act(int M, int N, int K, double alpha, const uint16_t *A, int lda,
                           const uint16_t *B, int ldb, const float *bias, int act, double *ref,
                           double *den, int threads) {
  half_gemm(oracle_bf16_to_double, M, N, K, alpha, A, lda, B, ldb, bias, act, ref, den, threads);
}

void oracle_bgemm_entries(int K, double alpha, const uint16_t *A, int lda, const uint16_t *B,
                          int ldb, const float *bias, int act, const int64_t *rows,
                          const int64_t *cols, int64_t count, double *ref, double *den,
                          int threads) {
  half_entries(oracle_bf16_to_double, K, alpha, A, lda, B, ldb, bias, act, rows, cols, count, ref,
               den, threads);
}

int oracle_max_threads(void) { return oracle_threads(0); }
