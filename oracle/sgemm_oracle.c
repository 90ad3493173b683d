/*
 * CPU oracle for row-major single-precision GEMM.  TEST INFRASTRUCTURE ONLY:
 * the parity tests, the smoke check and the benchmark's CPU-baseline leg call
 * it; the GPU library never links, loads or calls anything here, and nothing
 * here uses a HIP header or shares code with the GPU path.
 *
 * What it computes is the plain definition of the operation, written out:
 *
 *     C_out(i,j) = alpha * sum_{k=0}^{K-1} A(i,k) * B(k,j)  +  beta * C_in(i,j)
 *
 * for 0 <= i < M, 0 <= j < N, with A an M x K matrix, B a K x N matrix and
 * C an M x N matrix ("Deep dive into the sgemmNN algorithm", lazypool-blog,
 * opening section: C = alpha*A*B + beta*C, A is m x k, B is k x n, C is
 * m x n).  Storage is row-major with leading dimensions, X(i,j) at
 * X[i*ldX + j]: the row-major one-thread-per-element kernels of the
 * naive-to-tiled tutorial pages (m.lqnn.cn/news/94381 section 1.1;
 * "GPU-accelerated matrix computation ..." section 3.1) index A[row*K+k] and
 * B[k*N+col], and the sgemmNN page adds the explicit lda/ldb/ldc arguments.
 *
 * Precision: every float product is exact in double (24+24 < 53 significant
 * bits); the K-term sum runs in double in sequential k order, so the oracle's
 * own error is at most about K * 2^-53 * sum_k |a_ik||b_kj|, far below the
 * float32 rounding of any GPU result.  The result is returned in double and is
 * never rounded to float.
 *
 * Readings where the pages are silent (each listed in the design notes):
 *   - beta == 0 means the beta term is absent: C_in is not read, so a NaN in
 *     C_in does not reach the output.
 *   - alpha == 0 or K == 0 means the product term is absent: A and B are not
 *     read and the result is beta * C_in (zero when beta == 0 as well).
 *   - Only the M x N window is defined; padding between the logical width and
 *     the leading dimension is never read.
 *
 * Parallelism: OpenMP splits the independent output rows i over threads.
 * Each output element is still one sequential k-loop; no sum is reordered.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Row i of the definition.  acc[0..N) receives alpha*sum_k A(i,k)B(k,j)
 * + beta*C_in(i,j) in double; absab (optional) receives sum_k |A(i,k)||B(k,j)|.
 * The loop order inside the row is k then j, so acc[j] still adds its K terms
 * in the order k = 0, 1, ..., K-1. */
static void oracle_row(int i, int N, int K, double alpha, const float* A, long lda,
                       const float* B, long ldb, double beta, const float* Cin, long ldc,
                       double* acc, double* absab) {
  const int product = (alpha != 0.0) && (K > 0);
  for (int j = 0; j < N; ++j) {
    acc[j] = 0.0;
    if (absab) absab[j] = 0.0;
  }
  if (product) {
    const float* a_row = A + (size_t)i * (size_t)lda;
    for (int k = 0; k < K; ++k) {
      const double a = (double)a_row[k];
      const float* b_row = B + (size_t)k * (size_t)ldb;
      for (int j = 0; j < N; ++j) acc[j] += a * (double)b_row[j];
      if (absab)
        for (int j = 0; j < N; ++j) absab[j] += fabs(a) * fabs((double)b_row[j]);
    }
  }
  for (int j = 0; j < N; ++j) {
    double v = product ? alpha * acc[j] : 0.0;
    if (beta != 0.0) v += beta * (double)Cin[(size_t)i * (size_t)ldc + j];
    acc[j] = v;
  }
}

/*
 * Full result.  Cout (and absab, when not NULL) are dense M x N double arrays
 * with row stride N.  Returns 0, or -1 on a negative size.  nthreads <= 0
 * uses the OpenMP default.
 */
int oracle_sgemm_rm(int M, int N, int K, double alpha, const float* A, long lda, const float* B,
                    long ldb, double beta, const float* Cin, long ldc, double* Cout,
                    double* absab, int nthreads) {
  if (M < 0 || N < 0 || K < 0) return -1;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
#pragma omp parallel for schedule(static)
  for (int i = 0; i < M; ++i)
    oracle_row(i, N, K, alpha, A, lda, B, ldb, beta, Cin, ldc, Cout + (size_t)i * N,
               absab ? absab + (size_t)i * N : NULL);
  return 0;
}

/*
 * Selected entries only: for e in [0, count), out[e] and absab[e] receive the
 * definition at (rows[e], cols[e]).  Used for parity at sizes where the full
 * result is too slow on the CPU.  Returns 0, or -1 on a bad index.
 */
int oracle_sgemm_rm_entries(int M, int N, int K, double alpha, const float* A, long lda,
                            const float* B, long ldb, double beta, const float* Cin, long ldc,
                            const int64_t* rows, const int64_t* cols, long count, double* out,
                            double* absab, int nthreads) {
  for (long e = 0; e < count; ++e)
    if (rows[e] < 0 || rows[e] >= M || cols[e] < 0 || cols[e] >= N) return -1;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
  const int product = (alpha != 0.0) && (K > 0);
#pragma omp parallel for schedule(static)
  for (long e = 0; e < count; ++e) {
    const size_t i = (size_t)rows[e], j = (size_t)cols[e];
    double s = 0.0, sa = 0.0;
    if (product)
      for (int k = 0; k < K; ++k) {
        const double a = (double)A[i * (size_t)lda + k];
        const double b = (double)B[(size_t)k * (size_t)ldb + j];
        s += a * b;
        sa += fabs(a) * fabs(b);
      }
    double v = product ? alpha * s : 0.0;
    if (beta != 0.0) v += beta * (double)Cin[i * (size_t)ldc + j];
    out[e] = v;
    if (absab) absab[e] = sa;
  }
  return 0;
}
