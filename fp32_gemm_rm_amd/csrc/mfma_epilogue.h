// MFMA SGEMM, tile epilogues: alpha/beta on C in batches of loads before stores, the
// accumulator-to-C mapping of a wavefront, and the in-tile K-split reduction.
#pragma once

#include "mfma_operand.h"

namespace sgemm_impl {
namespace mfma_detail {

// C := alpha * x[u] + beta * C at the NV elements (row(u), col(u)) of this lane, given
// by coord(u, row, col); C is not read when beta == 0.  GUARD (bit 0: rows, bit 1:
// columns): elements past M or N are skipped.  Every C value of the batch is loaded
// before the first store: a load after a store into the same array would wait for that
// store (the compiler cannot tell
// that the addresses differ), which turns the epilogue into a chain of round trips.
template <int NV, int GUARD, typename Coord>
__device__ __forceinline__ void finish_c(const Problem& p, const float (&x)[NV], Coord coord) {
  auto inside = [&](int row, int col) { return (!(GUARD & 1) || row < p.M) && (!(GUARD & 2) || col < p.N); };
  if (p.beta == 0.0f) {
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      int row, col;
      coord(u, row, col);
      if (inside(row, col)) p.C[(long long)row * p.ldc + col] = p.alpha * x[u];
    }
    return;
  }
  float c[NV];
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    int row, col;
    coord(u, row, col);
    c[u] = inside(row, col) ? p.C[(long long)row * p.ldc + col] : 0.f;
  }
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    int row, col;
    coord(u, row, col);
    if (inside(row, col)) p.C[(long long)row * p.ldc + col] = fmaf(p.alpha, x[u], p.beta * c[u]);
  }
}

// The accumulators of one wavefront (FM x FN blocks of 32 x 32 at (m0 + wm0, n0 + wn0))
// to C, one row of blocks at a time, or raw to a stream-K partial tile `part`.
// Register r of lane l is row 8*(r/4) + 4*lh + r%4, column lr of its block.
template <int BM, int BN, int FM, int FN, int GUARD>
__device__ __forceinline__ void store_acc(const Problem& p, const v16f (&acc)[FM][FN], int m0, int n0, int wm0,
                                          int wn0, int lr, int lh, float* part) {
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    float x[FN * 16];
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) x[j * 16 + r] = acc[i][j][r];
    auto coord = [&](int u, int& row, int& col) {
      const int j = u / 16, r = u % 16;
      row = m0 + wm0 + i * 32 + 8 * (r / 4) + 4 * lh + (r % 4);
      col = n0 + wn0 + j * 32 + lr;
    };
    if (part != nullptr) {  // stream-K partial tile (full tiles only)
#pragma unroll
      for (int u = 0; u < FN * 16; ++u) {
        int row, col;
        coord(u, row, col);
        part[(row - m0) * BN + (col - n0)] = x[u];
      }
      continue;
    }
    finish_c<FN * 16, GUARD>(p, x, coord);
  }
}

// The end of a tile: with no K split, store_acc; with KS > 1 the KS wavefronts of one
// output block pass their partial sums through LDS (free after the K loop's last
// barrier); then each of them finishes 1/KS of the block's accumulator registers,
// adding the partials in the fixed order 0, 1, ..., KS-1, so that the epilogue's C
// traffic is spread over all wavefronts.
template <int BM, int BN, int WM, int WN, int KS, int FM, int FN, int GUARD>
__device__ __forceinline__ void finish_acc(const Problem& p, const v16f (&acc)[FM][FN], float* smem, int m0, int n0,
                                           float* part) {
  const int w = threadIdx.x / 64, l = threadIdx.x % 64;
  const int lr = l % 32, lh = l / 32;
  // K-group and spatial position of this wavefront (compile-time zero K-group without a
  // K split, which keeps the fragment-read addresses foldable)
  const int ks = KS == 1 ? 0 : w / (WM * WN), sp = KS == 1 ? w : w % (WM * WN);
  const int wm0 = (sp / WN) * (BM / WM), wn0 = (sp % WN) * (BN / WN);
  if constexpr (KS == 1) {
    store_acc<BM, BN, FM, FN, GUARD>(p, acc, m0, n0, wm0, wn0, lr, lh, part);
  } else {
    // register r of lane l is row 8*(r/4) + 4*lh + r%4, column lr of its 32 x 32 block
    constexpr int kSlots = FM * FN * 16;      // accumulator registers per lane
    constexpr int kPart = kSlots * 64;        // floats per wavefront
    constexpr int kStride = WM * WN * kPart;  // between the partials of consecutive K-groups
    static_assert(kSlots % KS == 0, "registers split evenly over the K-groups");
    float* mine = smem + (ks * (WM * WN) + sp) * kPart + l;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) mine[((i * FN + j) * 16 + r) * 64] = acc[i][j][r];
    __syncthreads();
    const float* sums = smem + sp * kPart + l;
    constexpr int kMine = kSlots / KS;
    float x[kMine];
#pragma unroll
    for (int u = 0; u < kMine; ++u) {
      const int s = ks * kMine + u;  // register (i, j, r) = (s / (16 FN), (s / 16) % FN, s % 16)
      x[u] = sums[s * 64];
#pragma unroll
      for (int q = 1; q < KS; ++q) x[u] += sums[q * kStride + s * 64];
    }
    auto coord = [&](int u, int& row, int& col) {
      const int s = ks * kMine + u, i = s / (FN * 16), j = (s / 16) % FN, r = s % 16;
      row = m0 + wm0 + i * 32 + 8 * (r / 4) + 4 * lh + (r % 4);
      col = n0 + wn0 + j * 32 + lr;
    };
    if (part != nullptr) {  // stream-K partial tile (full tiles only)
#pragma unroll
      for (int u = 0; u < kMine; ++u) {
        int row, col;
        coord(u, row, col);
        part[(row - m0) * BN + (col - n0)] = x[u];
      }
      return;
    }
    finish_c<kMine, GUARD>(p, x, coord);
  }
}

}  // namespace mfma_detail
}  // namespace sgemm_impl
