// LDS-tiled SGEMM with 128-bit global loads (m.lqnn.cn/news/94381 sections 2-5:
// shared-memory tiles, zero-filled edge loads, +1 row padding, float4 loads and
// four independent accumulators per thread; mlqm.cn/news/1180856 sections 4.2-4.3).
//
// Tile: 32 x 32 outputs, K in steps of 32, 256 threads (four 64-lane
// wavefronts).  Thread t owns the four adjacent outputs C[ty][4tx .. 4tx+3] with
// tx = t % 8, ty = t / 8, so a wavefront spans 8 rows x 32 columns.
//
// LDS layout on gfx950:
//   As[32][33]: A tile, row-major, one word of padding per row.  In the inner
//     loop a wavefront reads As[ty][k] for 8 distinct rows ty; with the 33-word
//     stride those 8 words fall in 8 distinct banks (stride 32 would put them in
//     at most 2), and each word is broadcast to the 8 lanes sharing the row.
//   Bs[32][32]: B tile, row-major, unpadded: a wavefront reads one float4
//     Bs[k][4tx] per lane, i.e. 8 distinct 16-byte words of one row, broadcast.
//
// Global loads: each thread loads one float4 of A (row t/8, k = 4*(t%8)) and one
// of B (row t/8, columns 4*(t%8)); 8 lanes cover 128 contiguous bytes of a row.
// Elements outside M, N or K are loaded as zero, which keeps the inner loop free
// of branches.  The 128-bit path needs 16-byte aligned rows (base pointer and
// leading dimension); otherwise the kernel is instantiated with scalar loads.
#include "internal.h"

namespace sgemm_impl {
namespace {

constexpr int T = 32;

template <bool VEC>
__device__ __forceinline__ float4 load4_guarded(const float* base, long long ld, int r, int c0, int rows, int cols) {
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  if (r >= rows) return v;
  const float* p = base + (long long)r * ld + c0;
  if (VEC && c0 + 3 < cols) return *reinterpret_cast<const float4*>(p);
  if (c0 + 0 < cols) v.x = p[0];
  if (c0 + 1 < cols) v.y = p[1];
  if (c0 + 2 < cols) v.z = p[2];
  if (c0 + 3 < cols) v.w = p[3];
  return v;
}

// TA / TB: A stored K x M (element (i, k) at A[k*lda + i]) / B stored N x K.  A
// transposed operand is read with the same coalesced float4 loads along its
// contiguous dimension, and the four values are written down a column of the
// As[m][k] / Bs[k][n] tile instead of along a row.  Into the unpadded Bs those column
// stores conflict (the 8 lanes of a row share a bank); this stage keeps the pages'
// tile layout, and the orientations are tuned in the MFMA kernel instead.
template <bool VEC, bool TA, bool TB>
__global__ __launch_bounds__(256) void lds_tiled_kernel(Problem p, int col_blocks) {
  p = batch_entry(p);
  __shared__ __attribute__((aligned(16))) float As[T][T + 1];
  __shared__ __attribute__((aligned(16))) float Bs[T][T];
  poison_lds(&As[0][0], T * (T + 1));
  poison_lds(&Bs[0][0], T * T);
  const int t = threadIdx.x;
  const int tx = t % 8, ty = t / 8;
  const int bm = blockIdx.x / col_blocks;
  const int bn = blockIdx.x - bm * col_blocks;
  const int m0 = bm * T, n0 = bn * T;
  const float* A = TA ? p.A + m0 : p.A + (long long)m0 * p.lda;
  const float* B = TB ? p.B + (long long)n0 * p.ldb : p.B + n0;
  const int rows_left = p.M - m0, cols_left = p.N - n0;

  float acc0 = 0.f, acc1 = 0.f, acc2 = 0.f, acc3 = 0.f;
  for (int k0 = 0; k0 < p.K; k0 += T) {
    if (TA) {  // a = A(m0 + 4tx .. 4tx+3, k0 + ty)
      const float4 a = load4_guarded<VEC>(A + (long long)k0 * p.lda, p.lda, ty, 4 * tx, p.K - k0, rows_left);
      As[4 * tx + 0][ty] = a.x;
      As[4 * tx + 1][ty] = a.y;
      As[4 * tx + 2][ty] = a.z;
      As[4 * tx + 3][ty] = a.w;
    } else {  // a = A(m0 + ty, k0 + 4tx .. 4tx+3)
      const float4 a = load4_guarded<VEC>(A + k0, p.lda, ty, 4 * tx, rows_left, p.K - k0);
      As[ty][4 * tx + 0] = a.x;
      As[ty][4 * tx + 1] = a.y;
      As[ty][4 * tx + 2] = a.z;
      As[ty][4 * tx + 3] = a.w;
    }
    if (TB) {  // b = B(k0 + 4tx .. 4tx+3, n0 + ty)
      const float4 b = load4_guarded<VEC>(B + k0, p.ldb, ty, 4 * tx, cols_left, p.K - k0);
      Bs[4 * tx + 0][ty] = b.x;
      Bs[4 * tx + 1][ty] = b.y;
      Bs[4 * tx + 2][ty] = b.z;
      Bs[4 * tx + 3][ty] = b.w;
    } else {  // b = B(k0 + ty, n0 + 4tx .. 4tx+3)
      *reinterpret_cast<float4*>(&Bs[ty][4 * tx]) =
          load4_guarded<VEC>(B + (long long)k0 * p.ldb, p.ldb, ty, 4 * tx, p.K - k0, cols_left);
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < T; ++k) {
      const float av = As[ty][k];
      const float4 bv = *reinterpret_cast<const float4*>(&Bs[k][4 * tx]);
      acc0 = fmaf(av, bv.x, acc0);
      acc1 = fmaf(av, bv.y, acc1);
      acc2 = fmaf(av, bv.z, acc2);
      acc3 = fmaf(av, bv.w, acc3);
    }
    __syncthreads();  // the next iteration overwrites the tiles
  }

  if (ty >= rows_left) return;
  float* c = p.C + (long long)(m0 + ty) * p.ldc + n0 + 4 * tx;
  const float accs[4] = {acc0, acc1, acc2, acc3};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if (4 * tx + e < cols_left) {
      c[e] = (p.beta == 0.0f) ? p.alpha * accs[e] : fmaf(p.alpha, accs[e], p.beta * c[e]);
    }
  }
}

}  // namespace

hipError_t launch_lds_tiled(const Problem& p, int batch, hipStream_t stream) {
  const long long cb = (p.N + T - 1) / T;
  const long long rb = (p.M + T - 1) / T;
  if (!grid_fits(cb * rb, 256)) return hipErrorInvalidConfiguration;
  const bool vec = vec_loads_ok(p, batch);
  const dim3 grid((unsigned)(cb * rb), batch), block(256);
#define SGEMM_LAUNCH_TILED(V, TA_, TB_) \
  hipLaunchKernelGGL((lds_tiled_kernel<V, TA_, TB_>), grid, block, 0, stream, p, (int)cb)
  if (vec) {
    if (p.ta && p.tb) SGEMM_LAUNCH_TILED(true, true, true);
    else if (p.ta) SGEMM_LAUNCH_TILED(true, true, false);
    else if (p.tb) SGEMM_LAUNCH_TILED(true, false, true);
    else SGEMM_LAUNCH_TILED(true, false, false);
  } else {
    if (p.ta && p.tb) SGEMM_LAUNCH_TILED(false, true, true);
    else if (p.ta) SGEMM_LAUNCH_TILED(false, true, false);
    else if (p.tb) SGEMM_LAUNCH_TILED(false, false, true);
    else SGEMM_LAUNCH_TILED(false, false, false);
  }
#undef SGEMM_LAUNCH_TILED
  return hipGetLastError();
}

}  // namespace sgemm_impl
