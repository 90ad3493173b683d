// MFMA SGEMM, tile epilogues: alpha/beta on C in batches of loads before stores, the
// accumulator-to-C mapping of a wavefront, and the in-tile K-split reduction.
#pragma once

#include "mfma_operand.h"

namespace sgemm_impl {
namespace mfma_detail {

// The C values at the NV elements (row(u), col(u)) of this lane, given by coord(u, row,
// col), into c; nothing is read when beta == 0.  Elements past M or N (GUARD bit 0: rows,
// bit 1: columns), which are not stored, read C's first element instead: the loads stay
// unconditional, with nothing that uses their values before the epilogue (a masked load
// followed by a select makes the compiler wait for every load in flight right there).
template <int NV, int GUARD, typename Coord>
__device__ __forceinline__ void load_c(const Problem& p, float (&c)[NV], Coord coord) {
  if (p.beta == 0.0f) return;
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    int row, col;
    coord(u, row, col);
    const bool inside = (!(GUARD & 1) || row < p.M) && (!(GUARD & 2) || col < p.N);
    c[u] = p.C[inside ? (long long)row * p.ldc + col : 0];
  }
}

// C := alpha * x[u] + beta * C at the same elements; elements past M or N (GUARD) are
// skipped.  Every C value is loaded (load_c) before the first store: a load after a store
// into the same array would wait for that store (the compiler cannot tell that the
// addresses differ), which turns the epilogue into a chain of round trips.  c: NV floats
// of the caller's for the loaded values.
template <int NV, int GUARD, typename Coord>
__device__ __forceinline__ void finish_c(const Problem& p, const float (&x)[NV], Coord coord, float (&c)[NV]) {
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
  load_c<NV, GUARD>(p, c, coord);
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    int row, col;
    coord(u, row, col);
    if (inside(row, col)) p.C[(long long)row * p.ldc + col] = fmaf(p.alpha, x[u], p.beta * c[u]);
  }
}

template <int V>
using fvec = float __attribute__((ext_vector_type(V)));

// finish_c for V adjacent columns per element: x[u] holds columns col(u) .. col(u) + V - 1.
// vec (the caller's uniform choice): C's rows and leading dimension are V-float aligned and, with GUARD bit 1, N is a
// multiple of V (a vector is then wholly inside or wholly past N): each element is read
// and written as one V-float vector; otherwise component by component, each guarded.
template <int NV, int V, int GUARD, bool vec, typename Coord>
__device__ __forceinline__ void finish_c_vec(const Problem& p, const fvec<V> (&x)[NV], Coord coord) {
  auto inside = [&](int row, int col) { return (!(GUARD & 1) || row < p.M) && (!(GUARD & 2) || col < p.N); };
  auto at = [&](int row, int col) { return p.C + (long long)row * p.ldc + col; };
  auto put = [&](int row, int col, const fvec<V>& v) {
    if constexpr (vec) {
      if (inside(row, col)) *reinterpret_cast<fvec<V>*>(at(row, col)) = v;
    } else {
#pragma unroll
      for (int e = 0; e < V; ++e)
        if (inside(row, col + e)) at(row, col)[e] = v[e];
    }
  };
  if (p.beta == 0.0f) {
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      int row, col;
      coord(u, row, col);
      put(row, col, p.alpha * x[u]);
    }
    return;
  }
  fvec<V> c[NV];
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    int row, col;
    coord(u, row, col);
    if constexpr (vec) {
      c[u] = inside(row, col) ? *reinterpret_cast<const fvec<V>*>(at(row, col)) : fvec<V>(0.f);
    } else {
#pragma unroll
      for (int e = 0; e < V; ++e) c[u][e] = inside(row, col + e) ? at(row, col)[e] : 0.f;
    }
  }
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    int row, col;
    coord(u, row, col);
    put(row, col, p.alpha * x[u] + p.beta * c[u]);
  }
}

// Output (row, column) of register r of lane (lr, lh) in block (i, j) of a wavefront
// whose tile starts at (r0, c0): the MFMA puts it at row 8*(r/4) + 4*lh + r%4 and column
// lr of the block, i.e. at the A line and B line of those lanes (frag_line).
template <int VA, int VB>
__device__ __forceinline__ void acc_coord(int i, int j, int r, int lr, int lh, int r0, int c0, int& row, int& col) {
  row = r0 + frag_line<VA>(i, 8 * (r / 4) + 4 * lh + (r % 4));
  col = c0 + frag_line<VB>(j, lr);
}

// The accumulators of one wavefront (FM x FN blocks of 32 x 32 at (m0 + wm0, n0 + wn0))
// to C, one row of blocks at a time, or raw to a stream-K partial tile `part`.
// With B's lines in groups of VB = 4 (frag_line), a lane holds 4 adjacent columns of
// each of its rows and stores them as one 128-bit vector where C allows it: 32-bit stores
// 16 bytes apart across the lanes cost 4x the cache-line writes (4096^3 on 256 x 256
// tiles: 972 against 929 us).  With VB = 2 the 64-bit stores serve launches of full tiles
// only (GUARD bit 2; 2048^3: 125.4 against 127.4 us); with partial tiles in the launch
// they made it slower (2000 x 1950 x 1000: 80.0 against 70.1 us).
template <int BM, int BN, int FM, int FN, int VA, int VB, int GUARD>
__device__ __forceinline__ void store_acc(const Problem& p, const v16f (&acc)[FM][FN], int m0, int n0, int wm0,
                                          int wn0, int lr, int lh, float* part) {
  if constexpr (VB == 4 || (VB == 2 && (GUARD & 4))) {
    // vector access to C (stream-K partial tiles, BN-float rows in a 16-byte aligned
    // workspace, always take it)
    const bool vec = (((reinterpret_cast<unsigned long long>(p.C) | (unsigned long long)p.ldc * 4) % (4 * VB)) == 0 &&
                      (!(GUARD & 2) || p.N % VB == 0));
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      constexpr int NV = FN / VB * 16;
      fvec<VB> x[NV];  // x[q * 16 + r]: register r of blocks VB q .. VB q + VB - 1
#pragma unroll
      for (int q = 0; q < FN / VB; ++q)
#pragma unroll
        for (int r = 0; r < 16; ++r)
#pragma unroll
          for (int v = 0; v < VB; ++v) x[q * 16 + r][v] = acc[i][VB * q + v][r];
      auto coord = [&](int u, int& row, int& col) {
        acc_coord<VA, VB>(i, VB * (u / 16), u % 16, lr, lh, m0 + wm0, n0 + wn0, row, col);
      };
      if (part != nullptr) {  // stream-K partial tile (full tiles only)
#pragma unroll
        for (int u = 0; u < NV; ++u) {
          int row, col;
          coord(u, row, col);
          *reinterpret_cast<fvec<VB>*>(part + (row - m0) * BN + (col - n0)) = x[u];
        }
        continue;
      }
      if (vec)  // uniform: one of two copies of the stores, not a branch per store
        finish_c_vec<NV, VB, GUARD, true>(p, x, coord);
      else
        finish_c_vec<NV, VB, GUARD, false>(p, x, coord);
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    float x[FN * 16];
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) x[j * 16 + r] = acc[i][j][r];
    auto coord = [&](int u, int& row, int& col) {
      acc_coord<VA, VB>(i, u / 16, u % 16, lr, lh, m0 + wm0, n0 + wn0, row, col);
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
    float c[FN * 16];
    finish_c<FN * 16, GUARD>(p, x, coord, c);
  }
}

// Output (row, column) of the u-th of the accumulator registers that a lane finishes after
// the K-split reduction of finish_acc (KS > 1): 1/KS of its wavefront's registers, chosen by
// its K-group.
template <int BM, int BN, int WM, int WN, int KS, int FM, int FN, int VA, int VB>
__device__ __forceinline__ void ksplit_coord(int u, int m0, int n0, int& row, int& col) {
  const int w = threadIdx.x / 64, l = threadIdx.x % 64;
  const int ks = w / (WM * WN), sp = w % (WM * WN);
  const int wm0 = (sp / WN) * (BM / WM), wn0 = (sp % WN) * (BN / WN);
  constexpr int kMine = FM * FN * 16 / KS;
  const int s = ks * kMine + u;  // register (i, j, r) = (s / (16 FN), (s / 16) % FN, s % 16)
  acc_coord<VA, VB>(s / (FN * 16), (s / 16) % FN, s % 16, l % 32, l / 32, m0 + wm0, n0 + wn0, row, col);
}

// The end of a tile: with no K split, store_acc; with KS > 1 the KS wavefronts of one
// output block pass their partial sums through LDS (free after the K loop's last
// barrier); then each of them finishes 1/KS of the block's accumulator registers,
// adding the partials in the fixed order 0, 1, ..., KS-1, so that the epilogue's C
// traffic is spread over all wavefronts.
template <int BM, int BN, int WM, int WN, int KS, int FM, int FN, int VA, int VB, int GUARD>
__device__ __forceinline__ void finish_acc(const Problem& p, const v16f (&acc)[FM][FN], float* smem, int m0, int n0,
                                           float* part) {
  const int w = threadIdx.x / 64, l = threadIdx.x % 64;
  const int lr = l % 32, lh = l / 32;
  // K-group and spatial position of this wavefront (compile-time zero K-group without a
  // K split, which keeps the fragment-read addresses foldable)
  const int ks = KS == 1 ? 0 : w / (WM * WN), sp = KS == 1 ? w : w % (WM * WN);
  const int wm0 = (sp / WN) * (BM / WM), wn0 = (sp % WN) * (BN / WN);
  if constexpr (KS == 1) {
    store_acc<BM, BN, FM, FN, VA, VB, GUARD>(p, acc, m0, n0, wm0, wn0, lr, lh, part);
  } else {
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
      const int s = ks * kMine + u;
      x[u] = sums[s * 64];
#pragma unroll
      for (int q = 1; q < KS; ++q) x[u] += sums[q * kStride + s * 64];
    }
    auto coord = [&](int u, int& row, int& col) {
      ksplit_coord<BM, BN, WM, WN, KS, FM, FN, VA, VB>(u, m0, n0, row, col);
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
    float c[kMine];
    finish_c<kMine, GUARD>(p, x, coord, c);
  }
}

}  // namespace mfma_detail
}  // namespace sgemm_impl
