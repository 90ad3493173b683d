// Naive SGEMM: one thread per element of C, reading A and B straight from
// global memory (m.lqnn.cn/news/94381 section 1.1; "GPU-accelerated matrix
// computation ..." section 3.1; mlqm.cn/news/1180856 section 4.1).
//
// gfx950 mapping: a workgroup is 64 x 4 threads, so one 64-lane wavefront
// covers 64 consecutive columns of one row.  Its B loads B[k*ldb + j] are one
// contiguous 256-byte segment per k and its A load A[i*lda + k] is the same
// address for the whole wavefront (a broadcast).  The kernel's limit is reuse,
// not coalescing: every k-step moves 2 floats per 2 FLOP.  With B stored
// transposed (N x K) the wavefront's B loads stride by ldb instead; the
// baseline keeps its one-thread-per-element form in every orientation.
#include "internal.h"

namespace sgemm_impl {
namespace {

constexpr int kNaiveCols = 64;  // one wavefront across columns
constexpr int kNaiveRows = 4;

// TA / TB: A stored K x M (element (i, k) at A[k*lda + i]) / B stored N x K.
// Block id q (0 <= q < blocks) covers rows 4*(q / col_blocks) .. +3 and columns
// 64*(q % col_blocks) .. +63; the grid is capped at kStrideBlocks and strides over the
// block ids, so the work-item count of the dispatch stays within 32 bits for any M x N.
template <bool TA, bool TB>
__global__ __launch_bounds__(kNaiveCols* kNaiveRows) void naive_kernel(Problem p, long long col_blocks,
                                                                       long long blocks) {
  p = batch_entry(p);
  const long long sa = TA ? p.lda : 1, sb = TB ? 1 : p.ldb;  // steps along k
  for (long long q = blockIdx.x; q < blocks; q += gridDim.x) {
    const long long bm = q / col_blocks;
    const long long bn = q - bm * col_blocks;
    const long long i = bm * kNaiveRows + threadIdx.y;
    const long long j = bn * kNaiveCols + threadIdx.x;
    if (i >= p.M || j >= p.N) continue;
    const float* a = TA ? p.A + i : p.A + i * p.lda;
    const float* b = TB ? p.B + j * p.ldb : p.B + j;
    float acc = 0.0f;
    for (int k = 0; k < p.K; ++k) acc = fmaf(a[k * sa], b[k * sb], acc);
    float* c = p.C + i * p.ldc + j;
    *c = (p.beta == 0.0f) ? p.alpha * acc : fmaf(p.alpha, acc, p.beta * *c);
  }
}

// C := beta*C (zeros when beta == 0, without reading C).  One thread per element, with
// the same block map and grid stride as naive_kernel.
__global__ __launch_bounds__(256) void scale_kernel(float* C, long long ldc, long long sC, int M, int N,
                                                    float beta, long long col_blocks, long long blocks) {
  C += blockIdx.y * sC;
  for (long long q = blockIdx.x; q < blocks; q += gridDim.x) {
    const long long bm = q / col_blocks;
    const long long bn = q - bm * col_blocks;
    const long long i = bm * 4 + threadIdx.y;
    const long long j = bn * 64 + threadIdx.x;
    if (i >= M || j >= N) continue;
    float* c = C + i * ldc + j;
    *c = (beta == 0.0f) ? 0.0f : beta * *c;
  }
}

// Blocks of the one-thread-per-element grid: capped at kStrideBlocks.
inline unsigned stride_grid(long long blocks) {
  return (unsigned)(blocks < kStrideBlocks ? blocks : kStrideBlocks);
}

}  // namespace

hipError_t launch_naive(const Problem& p, int batch, hipStream_t stream) {
  const long long cb = (p.N + kNaiveCols - 1) / kNaiveCols;
  const long long rb = (p.M + kNaiveRows - 1) / kNaiveRows;
  const long long blocks = cb * rb;
  const dim3 grid(stride_grid(blocks), batch), block(kNaiveCols, kNaiveRows);
  if (p.ta && p.tb)
    hipLaunchKernelGGL((naive_kernel<true, true>), grid, block, 0, stream, p, cb, blocks);
  else if (p.ta)
    hipLaunchKernelGGL((naive_kernel<true, false>), grid, block, 0, stream, p, cb, blocks);
  else if (p.tb)
    hipLaunchKernelGGL((naive_kernel<false, true>), grid, block, 0, stream, p, cb, blocks);
  else
    hipLaunchKernelGGL((naive_kernel<false, false>), grid, block, 0, stream, p, cb, blocks);
  return hipGetLastError();
}

hipError_t launch_scale(const Problem& p, int batch, hipStream_t stream) {
  const long long cb = (p.N + 63) / 64;
  const long long rb = (p.M + 3) / 4;
  const long long blocks = cb * rb;
  hipLaunchKernelGGL(scale_kernel, dim3(stride_grid(blocks), batch), dim3(64, 4), 0, stream, p.C, p.ldc, p.sC, p.M,
                     p.N, p.beta, cb, blocks);
  return hipGetLastError();
}

}  // namespace sgemm_impl
