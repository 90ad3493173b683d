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
        xv[S][u][0] = xo ? x.x : 0.f; xv[S][u][1] = xo ? x.y : 0.f;
        xv[S][u][2] = xo ? x.z : 0.f; xv[S][u][3] = xo ? x.w : 0.f;
        yv[S][u][0] = yo ? y.x : 0.f; yv[S][u][1] = yo ? y.y : 0.f;
        yv[S][u][2] = yo ? y.z : 0.f; yv[S][u][3] = yo ? y.w : 0.f;
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

// A right thin strip (columns [n0, n0 + w) of C, w < 16) fused into the MFMA tiles (the
// launch uses it in the 64 configuration, for operands stored row-major: A along k, B along
// n; written for any configuration whose K-tile gives each thread one B value): a separate
// thin-strip workgroup on a CU beside a tile takes that tile's MFMA, LDS and load
// slots for the strip's whole latency-bound K loop (1000 x 1030 x 999 on 64 x 64 tiles:
// 23.8 us, against 21.5 us for the 1024 columns of tiles alone).  Fused, tile (bm, bn)
// computes rows [bm BM + 4 bn, + 4) of the strip from the A rows its K-tiles already hold
// in LDS and the strip's columns of B, which the workgroup stages beside them (BK x 16
// floats per K-tile); that takes BM / 4 tile columns per tile row.  Per K-tile each thread
// loads one value of B's strip, stores it with the tile's LDS stores, reads its operands
// (SK values of one A row and of one strip column) with the tile's fragment reads one
// K-tile ahead, and adds SK products on the VALU during the next K-tile's MFMAs.  The SS
// k-slices of each output are added through LDS in slice order at the end.  The loads are
// unconditional (a masked load compiles to a branch whose join waits for every load in
// flight): columns past the strip load the last strip column and only reach outputs that
// are not stored; in the last, partial K-tile the rows past K load row K - 1 and are
// zeroed as they are stored, since their A values are zeros and a product 0 * Inf would
// otherwise be NaN.
template <int BK, int NT>
struct FusedStrip {
  static constexpr int SR = 4;              // strip rows per tile
  static constexpr int SS = NT / (SR * 16);  // k-slices per K-tile (one per thread role)
  static constexpr int SK = BK / SS;         // k per slice
  static constexpr int kStride = BK + 4;     // LDS row stride of one strip column (floats)
  static constexpr int kStageFloats = 16 * kStride;

  const float* bcol;  // load role: column n0 + min(t % 16, w - 1) of B at k = 0
  long long ldb;
  int kk, jl;         // load role: row kk = t / 16 of the K-tile, column jl = t % 16
  int i, j, s;        // compute role: strip row i, column j, k-slice s
  float reg[2];
  float a[2][SK], b[2][SK];
  float acc;
  float cval;  // C at this thread's output (threads t < 16 SR, load_c)

  __device__ __forceinline__ void init(const Problem& p, int n0, int w, int t) {
    static_assert(NT == BK * 16, "one staged B value per thread and K-tile");
    static_assert(SK % 4 == 0 && SK * SS == BK, "slices of whole 16-byte chunks");
    kk = t / 16;
    jl = t % 16;
    ldb = p.ldb;
    bcol = p.B + n0 + min(jl, w - 1);
    i = t % SR;
    j = (t / SR) % 16;
    s = t / (SR * 16);
    acc = 0.f;
  }
  // the strip's B values of a full K-tile at k0
  template <int SET>
  __device__ __forceinline__ void load_full(int k0) { reg[SET] = bcol[(long long)(k0 + kk) * ldb]; }
  // the last K-tile, kl < BK valid rows: rows past K read row K - 1, and store zeroes them
  // (a select right after the load would make the compiler wait for the load there)
  template <int SET>
  __device__ __forceinline__ void load_tail(int k0, int kl) {
    reg[SET] = bcol[(long long)(k0 + min(kk, kl - 1)) * ldb];
  }
  // a full K-tile's values to its LDS stage
  template <int SET>
  __device__ __forceinline__ void store(float* stage) const { stage[jl * kStride + kk] = reg[SET]; }
  // a K-tile with kl valid rows (kl >= BK: full)
  template <int SET>
  __device__ __forceinline__ void store(float* stage, int kl) const {
    stage[jl * kStride + kk] = kk < kl ? reg[SET] : 0.f;
  }
  // operands of this thread's slice: A row `row` of the tile's A stage (swizzled 16-byte
  // chunks, operand stored along k) and strip column j
  template <int S>
  __device__ __forceinline__ void read(const float* a_stage, const float* stage, int row) {
#pragma unroll
    for (int c = 0; c < SK / 4; ++c) {
      const float4 x = *reinterpret_cast<const float4*>(a_stage + swz_slot<BK>(row, s * SK / 4 + c));
      const float4 y = *reinterpret_cast<const float4*>(stage + j * kStride + s * SK + 4 * c);
      a[S][4 * c] = x.x; a[S][4 * c + 1] = x.y; a[S][4 * c + 2] = x.z; a[S][4 * c + 3] = x.w;
      b[S][4 * c] = y.x; b[S][4 * c + 1] = y.y; b[S][4 * c + 2] = y.z; b[S][4 * c + 3] = y.w;
    }
  }
  template <int S>
  __device__ __forceinline__ void fma() {
#pragma unroll
    for (int e = 0; e < SK; ++e) acc = fmaf(a[S][e], b[S][e], acc);
  }
  // the C value of this thread's output (rows [r0, r0 + rows), columns [n0, n0 + w);
  // threads t < 16 SR finish them), loaded before the tile's epilogue so that it arrives
  // meanwhile; unconditional: the other threads read C's first element and do not use it
  __device__ __forceinline__ void load_c(const Problem& p, int r0, int rows, int n0, int w, int t) {
    if (p.beta == 0.0f) return;
    const bool mine = t < SR * 16 && i < rows && j < w;
    cval = p.C[mine ? (long long)(r0 + i) * p.ldc + n0 + j : 0];
  }
  // after the K loop: this thread's slice sum to LDS (red: NT floats that no wavefront
  // reads any more), before a barrier that the caller provides
  __device__ __forceinline__ void stash(float* red, int t) const { red[t] = acc; }
  // after that barrier: the slices' sums in slice order, then C := alpha * sum + beta * C
  // on rows [r0, r0 + rows) and columns [n0, n0 + w); cval holds C (load_c)
  __device__ __forceinline__ void finish(const Problem& p, const float* red, int r0, int rows, int n0, int w,
                                         int t) const {
    if (t < SR * 16) {
      float x = red[t];
#pragma unroll
      for (int q = 1; q < SS; ++q) x += red[q * SR * 16 + t];
      if (i < rows && j < w) {
        float* c = p.C + (long long)(r0 + i) * p.ldc + n0 + j;
        *c = p.beta == 0.0f ? p.alpha * x : fmaf(p.alpha, x, p.beta * cval);
      }
    }
  }
};

}  // namespace mfma_detail
}  // namespace sgemm_impl
