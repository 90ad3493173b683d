// MFMA SGEMM, the strips past the MFMA tiles: scalar edge tiles (register-blocked VALU,
// 256 configuration) and thin strips (16 x 16 x 4 MFMA blocks beside the tiles).
#pragma once

#include <type_traits>
#include "mfma_operand.h"
#include "regblock_tile.h"

namespace sgemm_impl {
namespace mfma_detail {

// Scalar edge-tile path: one 32 x 32 register-blocked VALU tile per workgroup; the
// workgroup's NT/256 groups of 256 threads split its K range and add their partial
// sums through LDS in the fixed group order.
using EdgeTile = RegBlock<32, 32, 32, 2, 2, 256, 2, 8>;
constexpr int kEdge = 32;

template <int GROUPS, bool TA, bool TB, bool VEC>
__device__ __forceinline__ void edge_tile(const Problem& p, int m0, int n0, float* smem) {
  constexpr int BK = 32;
  const int g = threadIdx.x / 256, tid = threadIdx.x % 256;
  // every group runs the same number of K-steps (the block's barriers must match);
  // group g covers k in [g*span, g*span + span), clipped to K
  const int steps = (p.K + BK * GROUPS - 1) / (BK * GROUPS);
  const int span = steps * BK;
  const int kbeg = min(g * span, p.K);
  const int klen = min(span, p.K - kbeg);
  float acc[2][2];
  EdgeTile::template compute<VEC, true, TA, TB>(p, m0, n0, kbeg, klen, steps, smem + g * EdgeTile::kLdsFloats, tid,
                                                acc);
  if constexpr (GROUPS > 1) {
    float* red = smem;  // [GROUPS-1][4][256]; the stages are free after compute()'s last barrier
    if (g > 0)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[((g - 1) * 4 + i) * 256 + tid] = acc[i / 2][i % 2];
    __syncthreads();
    if (g > 0) return;
#pragma unroll 1
    for (int q = 1; q < GROUPS; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i / 2][i % 2] += red[((q - 1) * 4 + i) * 256 + tid];
  }
  EdgeTile::template store<true>(p, m0, n0, tid, acc);
}

// Thin strips (configurations with EDGE_MIN > 1): columns [lo, lo + width) of rows
// [first, first + nlines) when `cols`, else rows [lo, lo + width) of columns [first,
// first + nlines); width <= 16 (under EDGE_MIN for a strip, up to 16 for the whole
// blocks of the 16 configuration) and nlines <= 16.  A strip that thin would cost
// a whole MFMA tile row or column (on 64 x 64 tiles a 17th tile column turns one wave of
// tiles into two), so it runs beside the MFMA tiles as 16 x 16 blocks on
// v_mfma_f32_16x16x4_f32: each wavefront of the workgroup takes a K slice, every lane
// loads its two operands straight from global memory (clamped addresses, masked to zero
// outside the strip, so the loads are unconditional), and the wavefronts' partial blocks
// are added through LDS in wavefront order.  16x16x4 lane layout: lane l supplies
// X(l % 16, l / 16) and Y(l / 16, l % 16); accumulator register r of lane l holds
// D(4 * (l / 16) + r, l % 16).  D(i, j) is (line i, output j) when `cols`, (output i,
// line j) otherwise.
constexpr int kThinMax = 16;    // widest thin strip, and lines per workgroup
// Row stride (floats) of the thin strip's reduction buffer [wavefront][register][lane]: the
// final sums read, per half-wavefront, 16 lanes of register r and 16 of register r + 1, and
// a stride of 64 put both on the same 16 banks (2-way conflicts); 80 puts them 16 apart.
constexpr int kThinRedStride = 80;
template <int NT>
constexpr int thin_red_floats() { return NT / 64 * 4 * kThinRedStride; }
template <int NT, bool TA, bool TB, bool VEC>
__device__ __forceinline__ void thin_strip(const Problem& p, bool cols, int first, int nlines, int lo, int width,
                                           float* smem) {
  typedef float v4f __attribute__((ext_vector_type(4)));
  constexpr int W = NT / 64;
  static_assert(NT >= 256, "one thread per output of the 16 x 16 block in the final sums");
  // An operand stored along k (A, or B^T) is read as float4s of 4 consecutive k when its
  // rows are 16-byte aligned: lane quad kq takes k = kb + 4 kq + s in MFMA step s of each
  // group of 4 steps (16 k), so a lane's 4 values are adjacent.  The other operand (A^T,
  // or B) is read element by element, 16 adjacent values per row across the lanes.
  constexpr bool VX = VEC && !TA, VY = VEC && TB;
  const int t = threadIdx.x, wv = t / 64, l = t % 64, i16 = l % 16, kq = l / 16;
  // this lane's row of op(A) (X operand) and column of op(B) (Y operand), clamped
  const int nx = cols ? nlines : width, ny = cols ? width : nlines;
  const int am = (cols ? first : lo) + min(i16, nx - 1), bn = (cols ? lo : first) + min(i16, ny - 1);
  const bool x_in = i16 < nx, y_in = i16 < ny;
  const float* arow = TA ? p.A + am : p.A + (long long)am * p.lda;  // element k at arow[k * (TA ? lda : 1)]
  const float* bcol = TB ? p.B + (long long)bn * p.ldb : p.B + bn;  // element k at bcol[k * (TB ? 1 : ldb)]
  auto xk = [&](int k) { return TA ? arow[(long long)k * p.lda] : arow[k]; };
  auto yk = [&](int k) { return TB ? bcol[k] : bcol[(long long)k * p.ldb]; };
  // [0, K16) in groups of 16 k, each wavefront a contiguous slice of whole groups; the
  // last 0-15 k (the tail) are one wavefront's extra steps.
  const int K16 = p.K & ~15;
  const int kc = ((K16 / 16 + W - 1) / W) * 16;
  const int k0 = min(wv * kc, K16), k1 = min(k0 + kc, K16);
  // The slice runs in chunks of U groups whose loads are issued one chunk ahead (two
  // register sets), so that a wavefront keeps up to 64 loads per lane in flight instead
  // of waiting out the memory latency every few steps; U = 4 for long slices, 1 for short
  // ones, whose groups past the slice would otherwise dominate.  Those groups (the last
  // chunks) load clamped addresses and contribute zeros.
  v4f acc = {0.f, 0.f, 0.f, 0.f};
  auto slice = [&](auto chunk) {
    constexpr int U = decltype(chunk)::value;
    float xv[2][U][4], yv[2][U][4];
    auto fetch = [&](auto set, int kbase) {
      constexpr int S = decltype(set)::value;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int kg = kbase + 16 * u;
        const bool kin = kg < k1;
        const int kl = min(kg, K16 - 16) + 4 * kq;  // inside [0, K16)
        float4 x, y;
        if (VX)
          x = *reinterpret_cast<const float4*>(arow + kl);
        else
          x = make_float4(xk(kl), xk(kl + 1), xk(kl + 2), xk(kl + 3));
        if (VY)
          y = *reinterpret_cast<const float4*>(bcol + kl);
        else
          y = make_float4(yk(kl), yk(kl + 1), yk(kl + 2), yk(kl + 3));
        const bool xo = x_in && kin, yo = y_in && kin;
        xv[S][u][0] = xo ? x.x : 0.f; xv[S][u][1] = xo ? x.y : 0.f; xv[S][u][2] = xo ? x.z : 0.f; xv[S][u][3] = xo ? x.w : 0.f;
        yv[S][u][0] = yo ? y.x : 0.f; yv[S][u][1] = yo ? y.y : 0.f; yv[S][u][2] = yo ? y.z : 0.f; yv[S][u][3] = yo ? y.w : 0.f;
      }
    };
    auto steps = [&](auto set) {
      constexpr int S = decltype(set)::value;
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xv[S][u][q], yv[S][u][q], acc, 0, 0, 0);
    };
    using Set0 = std::integral_constant<int, 0>;
    using Set1 = std::integral_constant<int, 1>;
    fetch(Set0{}, k0);
    for (int k = k0; k < k1; k += 32 * U) {
      fetch(Set1{}, k + 16 * U);
      steps(Set0{});
      fetch(Set0{}, k + 32 * U);
      steps(Set1{});
    }
  };
  if (K16 > 0) {
    if (k1 - k0 >= 16 * 16)  // 16 groups or more
      slice(std::integral_constant<int, 4>{});
    else
      slice(std::integral_constant<int, 1>{});
  }
  if (wv == W - 1 && K16 < p.K) {  // the tail: k = K16 + 4 u + kq in step u
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int kx = K16 + 4 * u + kq, kcl = min(kx, p.K - 1);
      const float av = xk(kcl), bv = yk(kcl);
      const bool kin = kx < p.K;
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x_in && kin ? av : 0.f, y_in && kin ? bv : 0.f, acc, 0, 0, 0);
    }
  }
  float* red = smem;  // [wavefront][register][lane], thin_red_floats<NT>() floats
#pragma unroll
  for (int r = 0; r < 4; ++r) red[(wv * 4 + r) * kThinRedStride + l] = acc[r];
  __syncthreads();
  if (t < 256) {
    const int i = t / 16, j = t % 16, lane = 16 * (i / 4) + j, r = i % 4;
    const int line = cols ? i : j, out = cols ? j : i;
    if (line < nlines && out < width) {
      float x = red[r * kThinRedStride + lane];
#pragma unroll
      for (int q = 1; q < W; ++q) x += red[(q * 4 + r) * kThinRedStride + lane];
      const int row = cols ? first + line : lo + out, col = cols ? lo + out : first + line;
      float* c = p.C + (long long)row * p.ldc + col;
      *c = p.beta == 0.0f ? p.alpha * x : fmaf(p.alpha, x, p.beta * *c);
    }
  }
}

}  // namespace mfma_detail
}  // namespace sgemm_impl
