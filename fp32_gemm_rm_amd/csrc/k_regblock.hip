// Register-blocked, double-buffered SGEMM on the vector ALU (the tile itself is
// in regblock_tile.h): 128 x 128 tiles with 8 x 8 outputs per thread when the
// problem has enough of them to fill the chip, otherwise 64 x 64 tiles with
// 4 x 4 outputs per thread.  256 threads per workgroup.  Full tiles take the
// unchecked path; tiles that reach past M or N take the bounds-checked one.
#include "regblock_tile.h"

namespace sgemm_impl {
namespace {

template <int BM, int BN, int BK, int TM, int TN, int PAD_A, bool VEC, bool TA, bool TB>
__global__ __launch_bounds__(256) void regblock_kernel(Problem p, int col_blocks) {
  p = batch_entry(p);
  using RB = RegBlock<BM, BN, BK, TM, TN, 256, PAD_A>;
  __shared__ __attribute__((aligned(16))) float lds[RB::kLdsFloats];
  poison_lds(lds, RB::kLdsFloats);
  const int bm = blockIdx.x / col_blocks;
  const int bn = blockIdx.x - bm * col_blocks;
  const int m0 = bm * BM, n0 = bn * BN;
  if (m0 + BM <= p.M && n0 + BN <= p.N)
    RB::template tile<VEC, false, TA, TB>(p, m0, n0, lds, threadIdx.x);
  else
    RB::template tile<VEC, true, TA, TB>(p, m0, n0, lds, threadIdx.x);
}

template <int BM, int BN, int BK, int TM, int TN, int PAD_A>
hipError_t launch_cfg(const Problem& p, int batch, hipStream_t stream) {
  const long long cb = (p.N + BN - 1) / BN;
  const long long rb = (p.M + BM - 1) / BM;
  if (!grid_fits(cb * rb, 256)) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)(cb * rb), batch), block(256);
  const bool vec = vec_loads_ok(p, batch);
#define SGEMM_LAUNCH_RB(V, TA_, TB_) \
  hipLaunchKernelGGL((regblock_kernel<BM, BN, BK, TM, TN, PAD_A, V, TA_, TB_>), grid, block, 0, stream, p, (int)cb)
  if (vec) {
    if (p.ta && p.tb) SGEMM_LAUNCH_RB(true, true, true);
    else if (p.ta) SGEMM_LAUNCH_RB(true, true, false);
    else if (p.tb) SGEMM_LAUNCH_RB(true, false, true);
    else SGEMM_LAUNCH_RB(true, false, false);
  } else {
    if (p.ta && p.tb) SGEMM_LAUNCH_RB(false, true, true);
    else if (p.ta) SGEMM_LAUNCH_RB(false, true, false);
    else if (p.tb) SGEMM_LAUNCH_RB(false, false, true);
    else SGEMM_LAUNCH_RB(false, false, false);
  }
#undef SGEMM_LAUNCH_RB
  return hipGetLastError();
}

}  // namespace

hipError_t launch_regblock(const Problem& p, int batch, hipStream_t stream) {
  const long long tiles128 = (long long)((p.M + 127) / 128) * ((p.N + 127) / 128) * batch;
  if (tiles128 >= 512) return launch_cfg<128, 128, 8, 8, 8, 4>(p, batch, stream);
  return launch_cfg<64, 64, 16, 4, 4, 4>(p, batch, stream);
}

}  // namespace sgemm_impl
