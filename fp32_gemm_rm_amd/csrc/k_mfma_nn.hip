// MFMA SGEMM instantiated for op(A) = A, op(B) = B (see mfma_gemm.h).
#include "mfma_gemm.h"

namespace sgemm_impl {

hipError_t launch_mfma_nn(const Problem& p, int batch, hipStream_t stream, int tiles, float* ws,
                           int slices) {
  return mfma_detail::launch_op<false, false>(p, batch, stream, tiles, ws, slices);
}

}  // namespace sgemm_impl
