// C-ABI entry points of libsgemm_rm: argument checks, the special cases,
// the choice of kernel family and the launches on the caller's stream.
// The operations and their return codes are specified in include/sgemm_rm.h.
#include "sgemm_rm.h"

#include "internal.h"

namespace {

using sgemm_impl::Problem;

// Checks shared by the single and the batched calls; positions are those of
// sgemm_rm (M N K alpha A lda B ldb beta C ldc).  Returns 0 or -(position).
int check_gemm(int M, int N, int K, float alpha, const float* A, int lda, const float* B, int ldb,
               const float* C, int ldc) {
  if (M < 0) return -1;
  if (N < 0) return -2;
  if (K < 0) return -3;
  const bool reads_ab = M > 0 && N > 0 && K > 0 && alpha != 0.0f;
  if (reads_ab && A == nullptr) return -5;
  if (lda < (K > 1 ? K : 1)) return -6;
  if (reads_ab && B == nullptr) return -7;
  if (ldb < (N > 1 ? N : 1)) return -8;
  if (M > 0 && N > 0 && C == nullptr) return -10;
  if (ldc < (N > 1 ? N : 1)) return -11;
  return 0;
}

// Enqueue `batch` problems spaced by p.sA, p.sB, p.sC (p already validated, M, N > 0).
int launch(Problem p, int batch, hipStream_t stream, int variant) {
  while (batch > 0) {
    const int chunk = batch < sgemm_impl::kMaxBatch ? batch : sgemm_impl::kMaxBatch;
    hipError_t err;
    if (p.alpha == 0.0f || p.K == 0) {
      if (p.beta == 1.0f) return 0;
      err = sgemm_impl::launch_scale(p, chunk, stream);
    } else {
      switch (variant) {
        case SGEMM_RM_VARIANT_NAIVE:
          err = sgemm_impl::launch_naive(p, chunk, stream);
          break;
        case SGEMM_RM_VARIANT_LDS_TILED:
          err = sgemm_impl::launch_lds_tiled(p, chunk, stream);
          break;
        case SGEMM_RM_VARIANT_REGBLOCK:
          err = sgemm_impl::launch_regblock(p, chunk, stream);
          break;
        case SGEMM_RM_VARIANT_MFMA:
        case SGEMM_RM_VARIANT_AUTO:
        default:
          err = sgemm_impl::launch_mfma(p, chunk, stream);
          break;
      }
    }
    if (err != hipSuccess) return (int)err;
    batch -= chunk;
    p.A += (long long)chunk * p.sA;
    p.B += (long long)chunk * p.sB;
    p.C += (long long)chunk * p.sC;
  }
  return 0;
}

int run(int M, int N, int K, float alpha, const float* A, int lda, const float* B, int ldb, float beta,
        float* C, int ldc, hipStream_t stream, int variant) {
  const int bad = check_gemm(M, N, K, alpha, A, lda, B, ldb, C, ldc);
  if (bad != 0) return bad;
  if (variant < SGEMM_RM_VARIANT_AUTO || variant > SGEMM_RM_VARIANT_MFMA) return -13;
  if (M == 0 || N == 0) return 0;
  const Problem p{M, N, K, alpha, beta, A, lda, B, ldb, C, ldc, 0, 0, 0};
  return launch(p, 1, stream, variant);
}

// Batched call: checks in parameter order of sgemm_rm_strided_batched
// (M N K alpha A lda strideA B ldb strideB beta C ldc strideC batch stream [variant]).
int run_batched(int M, int N, int K, float alpha, const float* A, int lda, long long sA, const float* B, int ldb,
                long long sB, float beta, float* C, int ldc, long long sC, int batch, hipStream_t stream,
                int variant) {
  if (M < 0) return -1;
  if (N < 0) return -2;
  if (K < 0) return -3;
  const bool any = M > 0 && N > 0 && batch > 0;
  const bool reads_ab = any && K > 0 && alpha != 0.0f;
  if (reads_ab && A == nullptr) return -5;
  if (lda < (K > 1 ? K : 1)) return -6;
  if (sA < 0) return -7;
  if (reads_ab && B == nullptr) return -8;
  if (ldb < (N > 1 ? N : 1)) return -9;
  if (sB < 0) return -10;
  if (any && C == nullptr) return -12;
  if (ldc < (N > 1 ? N : 1)) return -13;
  // the outputs of different batch entries must not overlap
  if (sC < 0 || (batch > 1 && M > 0 && N > 0 && sC < (long long)(M - 1) * ldc + N)) return -14;
  if (batch < 0) return -15;
  if (variant < SGEMM_RM_VARIANT_AUTO || variant > SGEMM_RM_VARIANT_MFMA) return -17;
  if (!any) return 0;
  const Problem p{M, N, K, alpha, beta, A, lda, B, ldb, C, ldc, sA, sB, sC};
  return launch(p, batch, stream, variant);
}

}  // namespace

extern "C" {

int sgemm_rm(int M, int N, int K, float alpha, const float* A, int lda, const float* B, int ldb, float beta,
             float* C, int ldc, hipStream_t stream) {
  return run(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, SGEMM_RM_VARIANT_AUTO);
}

int sgemm_rm_ex(int M, int N, int K, float alpha, const float* A, int lda, const float* B, int ldb, float beta,
                float* C, int ldc, hipStream_t stream, int variant) {
  return run(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, variant);
}

int sgemm_rm_strided_batched(int M, int N, int K, float alpha, const float* A, int lda, long long strideA,
                             const float* B, int ldb, long long strideB, float beta, float* C, int ldc,
                             long long strideC, int batch, hipStream_t stream) {
  return run_batched(M, N, K, alpha, A, lda, strideA, B, ldb, strideB, beta, C, ldc, strideC, batch, stream,
                     SGEMM_RM_VARIANT_AUTO);
}

int sgemm_rm_strided_batched_ex(int M, int N, int K, float alpha, const float* A, int lda, long long strideA,
                                const float* B, int ldb, long long strideB, float beta, float* C, int ldc,
                                long long strideC, int batch, hipStream_t stream, int variant) {
  return run_batched(M, N, K, alpha, A, lda, strideA, B, ldb, strideB, beta, C, ldc, strideC, batch, stream,
                     variant);
}

const char* sgemm_rm_strerror(int code) {
  static const char* const kInvalid[] = {
      "invalid argument 1",  "invalid argument 2",  "invalid argument 3",  "invalid argument 4",
      "invalid argument 5",  "invalid argument 6",  "invalid argument 7",  "invalid argument 8",
      "invalid argument 9",  "invalid argument 10", "invalid argument 11", "invalid argument 12",
      "invalid argument 13", "invalid argument 14", "invalid argument 15", "invalid argument 16",
      "invalid argument 17"};
  if (code == 0) return "success";
  if (code < 0 && code >= -17) return kInvalid[-code - 1];
  if (code > 0) return hipGetErrorString((hipError_t)code);
  return "unknown error code";
}

int sgemm_rm_version(void) { return 200; }

}  // extern "C"
