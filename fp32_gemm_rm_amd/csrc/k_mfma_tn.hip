// MFMA SGEMM instantiated for op(A) = A^T, op(B) = B (see mfma_gemm.h).
#include "mfma_gemm.h"

namespace sgemm_impl {

hipError_t launch_mfma_tn(const Problem& p, int batch, hipStream_t stream, int tiles, float* ws,
                           int slices) {
  return mfma_detail::launch_op<true, false>(p, batch, stream, tiles, ws, slices);
}

}  // namespace sgemm_impl
