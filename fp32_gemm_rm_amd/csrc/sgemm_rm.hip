// C-ABI entry points of libsgemm_rm: argument checks, the special cases,
// the choice of kernel family and the launches on the caller's stream.
// The operation and its return codes are specified in include/sgemm_rm.h.
#include "sgemm_rm.h"

#include "internal.h"

namespace {

using sgemm_impl::Problem;

// Argument checks in parameter order; returns 0 or -(1-based position).
int check_args(int M, int N, int K, float alpha, const float* A, int lda, const float* B, int ldb,
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

int run(int M, int N, int K, float alpha, const float* A, int lda, const float* B, int ldb, float beta,
        float* C, int ldc, hipStream_t stream, int variant) {
  const int bad = check_args(M, N, K, alpha, A, lda, B, ldb, C, ldc);
  if (bad != 0) return bad;
  if (variant < SGEMM_RM_VARIANT_AUTO || variant > SGEMM_RM_VARIANT_MFMA) return -13;
  if (M == 0 || N == 0) return 0;

  Problem p{M, N, K, alpha, beta, A, lda, B, ldb, C, ldc};
  hipError_t err;
  if (alpha == 0.0f || K == 0) {
    if (beta == 1.0f) return 0;
    err = sgemm_impl::launch_scale(p, stream);
  } else {
    switch (variant) {
      case SGEMM_RM_VARIANT_NAIVE:
        err = sgemm_impl::launch_naive(p, stream);
        break;
      case SGEMM_RM_VARIANT_LDS_TILED:
        err = sgemm_impl::launch_lds_tiled(p, stream);
        break;
      case SGEMM_RM_VARIANT_REGBLOCK:
        err = sgemm_impl::launch_regblock(p, stream);
        break;
      case SGEMM_RM_VARIANT_MFMA:
      case SGEMM_RM_VARIANT_AUTO:
      default:
        err = sgemm_impl::launch_mfma(p, stream);
        break;
    }
  }
  return err == hipSuccess ? 0 : (int)err;
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

const char* sgemm_rm_strerror(int code) {
  switch (code) {
    case 0: return "success";
    case -1: return "invalid argument 1: M < 0";
    case -2: return "invalid argument 2: N < 0";
    case -3: return "invalid argument 3: K < 0";
    case -5: return "invalid argument 5: A is NULL";
    case -6: return "invalid argument 6: lda < max(1, K)";
    case -7: return "invalid argument 7: B is NULL";
    case -8: return "invalid argument 8: ldb < max(1, N)";
    case -10: return "invalid argument 10: C is NULL";
    case -11: return "invalid argument 11: ldc < max(1, N)";
    case -13: return "invalid argument 13: unknown variant";
    default: break;
  }
  if (code > 0) return hipGetErrorString((hipError_t)code);
  return "unknown error code";
}

int sgemm_rm_version(void) { return 100; }

}  // extern "C"
