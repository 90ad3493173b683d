// MFMA SGEMM, operand staging: the LDS layouts of the A and B slices of a K-tile, their
// global loads (full, guarded and last K-tiles) and the MFMA fragment reads, and the
// per-configuration geometry.  The design is described at the top of mfma_gemm.h.
#pragma once

#include "internal.h"

namespace sgemm_impl {
namespace mfma_detail {

typedef float v16f __attribute__((ext_vector_type(16)));

// Word offset of X(row, 4*chunk) inside one LDS stage whose rows hold BK floats.
// 64 banks hold 16 chunks, i.e. max(1, 64/BK) rows; chunk indices are XORed with the
// row's index in units of that period (at most 16 distinct values), so 16 consecutive
// rows at one chunk, and 16/KC rows at all KC chunks, both land on 16 distinct chunk
// slots.
template <int BK>
__device__ __forceinline__ int swz_slot(int row, int chunk) {
  constexpr int kPeriod = BK >= 64 ? 1 : 64 / BK;
  constexpr int kMask = (BK / 4 > 16 ? 16 : BK / 4) - 1;
  return row * BK + 4 * (chunk ^ ((row / kPeriod) & kMask));
}

template <bool VEC>
__device__ __forceinline__ float4 load4(const float* p, int left) {
  if (left >= 4) {
    if (VEC) return *reinterpret_cast<const float4*>(p);
    return make_float4(p[0], p[1], p[2], p[3]);
  }
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  if (left > 0) v.x = p[0];
  if (left > 1) v.y = p[1];
  if (left > 2) v.z = p[2];
  return v;
}

// One MFMA operand of a K-tile: its R x BK slice (R = BM for A, BN for B) as the
// thread loads it from global memory, stores it in an LDS stage and reads it as
// MFMA fragments.  KROWS: the operand's rows in memory run along k (A, or B^T):
// the stage holds R rows of BK floats with swizzled 16-byte chunks and a fragment
// is two 128-bit reads.  Otherwise (A^T, or B) the stage holds BK rows of R floats
// with stride R + 4, and the fragments of V blocks (frag_line) are eight V-float reads.
// PACKED (rows along m or n, R >= 64; the LDS-DMA loads, which write 1 KiB runs): stride R
// instead, column c of k-row k at c ^ 32 in the k-rows 8-15 of every 16 (kslot): the
// fragment reads of k and k + 8 (the two lane halves) then fall on different banks, as the
// 4 padding words make them do otherwise.
template <int R, int BK, int NT, bool KROWS, bool PACKED = false>
struct Operand {
  static constexpr int KC = BK / 4;
  static constexpr int LOADS = R * BK / 4 / NT;  // float4 per thread per K-tile
  static constexpr int STRIDE = KROWS ? BK : PACKED ? R : R + 4;
  static constexpr int kStageFloats = KROWS ? R * BK : BK * STRIDE;
  static_assert(LOADS >= 1 && LOADS * NT * 4 == R * BK, "even load split");
  static_assert(!PACKED || (!KROWS && R >= 64), "packed rows along m or n, at least 64 floats");
  // word offset of X(line c, k) in a stage stored along m or n
  __device__ __forceinline__ static constexpr int kslot(int k, int c) {
    return k * STRIDE + (PACKED ? c ^ (((k >> 3) & 1) << 5) : c);
  }

  const float* base;  // element (r0, k = 0) of this tile's slice
  long long ld;
  int lim;                     // rows of the slice inside the matrix (R for a full tile)
  int row[LOADS], col[LOADS];  // KROWS: (r, chunk); else (k, 4 * r-quad)
  float4 reg[2][LOADS];  // two register sets for a prefetch distance of two K-tiles

  __device__ __forceinline__ void init(const float* X, long long ldx, int r0, int rows_left, int t) {
    ld = ldx;
    lim = rows_left < R ? rows_left : R;
    base = KROWS ? X + (long long)r0 * ldx : X + r0;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int q = t + i * NT;
      row[i] = KROWS ? q / KC : q / (R / 4);
      col[i] = KROWS ? q % KC : (q % (R / 4)) * 4;
    }
  }
  // full K-tile starting at k0.  GUARD: the slice may reach past the matrix (lim < R).
  // Every load is unconditional: a load under a branch makes the compiler wait for it
  // where the branches join, which would undo the prefetch of the guarded tiles.  A row
  // of A or B^T past the matrix (rows along k) is loaded from the last row; along r (rows
  // along m or n: B, or A^T) each element past the matrix is loaded from the last column.
  // Values past M or N only ever reach rows or columns of the product that are not stored
  // (output (i, j) takes row i of op(A) and column j of op(B) alone), so the clamped loads
  // only have to stay inside the matrix, and they are stored to LDS as loaded.  Along r the
  // limit is a multiple of 4 (launch_cfg leaves the last 1-3 rows or columns to the thin
  // strips), so no float4 straddles the edge, and one past it loads the last float4 inside.
  template <bool VEC, bool GUARD, int SET = 0>
  __device__ __forceinline__ void load_full(int k0) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      if (KROWS) {
        const int r = (!GUARD || row[i] < lim) ? row[i] : lim - 1;
        reg[SET][i] = load4<VEC>(base + (long long)r * ld + k0 + 4 * col[i], 4);
      } else {
        const int c = GUARD ? min(col[i], lim - 4) : col[i];
        reg[SET][i] = load4<VEC>(base + (long long)(k0 + row[i]) * ld + c, 4);
      }
    }
  }
  // global load instructions of one load_full
  static constexpr int kLoadInstrs(bool vec) { return vec ? LOADS : 4 * LOADS; }
  // last K-tile: kl = K - k0 < BK valid k; zeros past K (and past the matrix, GUARD)
  template <bool VEC, bool GUARD, int SET = 0>
  __device__ __forceinline__ void load_tail(int k0, int kl) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      if (KROWS)
        reg[SET][i] = (!GUARD || row[i] < lim)
                          ? load4<VEC>(base + (long long)row[i] * ld + k0 + 4 * col[i], kl - 4 * col[i])
                          : make_float4(0.f, 0.f, 0.f, 0.f);
      else if (row[i] >= kl)
        reg[SET][i] = make_float4(0.f, 0.f, 0.f, 0.f);
      else
        reg[SET][i] = GUARD ? load4<VEC>(base + (long long)(k0 + row[i]) * ld + col[i], lim - col[i])
                            : load4<VEC>(base + (long long)(k0 + row[i]) * ld + col[i], 4);
    }
  }
  // registers of set SET to an LDS stage
  template <int SET = 0>
  __device__ __forceinline__ void store(float* stage) const {
#pragma unroll
    for (int i = 0; i < LOADS; ++i)
      *reinterpret_cast<float4*>(stage + (KROWS ? swz_slot<BK>(row[i], col[i]) : kslot(row[i], col[i]))) =
          reg[SET][i];
  }
  // out[f0 + v][e] = X(c + v, 16g + 8lh + e), v < V, e = 0..7 (stage along m or n only):
  // the values of V blocks for the 8 MFMA steps of k-group g as V-float vectors (c is a
  // multiple of V, rows start on 16-byte boundaries)
  template <int V, int F>
  __device__ __forceinline__ static void read_vec(const float* stage, int c, int g, int lh, int f0,
                                                  float (&out)[F][8]) {
    static_assert(!KROWS && (V == 2 || V == 4), "vector fragment reads along m or n");
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float* q = stage + kslot(16 * g + 8 * lh + e, c);
      if constexpr (V == 4) {
        const float4 x = *reinterpret_cast<const float4*>(q);
        out[f0][e] = x.x; out[f0 + 1][e] = x.y; out[f0 + 2][e] = x.z; out[f0 + 3][e] = x.w;
      } else {
        const float2 x = *reinterpret_cast<const float2*>(q);
        out[f0][e] = x.x; out[f0 + 1][e] = x.y;
      }
    }
  }
  // out[e] = X(rr, 16g + 8lh + e), e = 0..7: this lane's values for the 8 MFMA steps of k-group g
  __device__ __forceinline__ static void read(const float* stage, int rr, int g, int lh, float (&out)[8]) {
    if constexpr (KROWS) {
      const float4 x0 = *reinterpret_cast<const float4*>(stage + swz_slot<BK>(rr, 4 * g + 2 * lh));
      const float4 x1 = *reinterpret_cast<const float4*>(stage + swz_slot<BK>(rr, 4 * g + 2 * lh + 1));
      out[0] = x0.x; out[1] = x0.y; out[2] = x0.z; out[3] = x0.w;
      out[4] = x1.x; out[5] = x1.y; out[6] = x1.z; out[7] = x1.w;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) out[e] = stage[kslot(16 * g + 8 * lh + e, rr)];
    }
  }
};

// Lanes and lines of a wavefront's F blocks along m (A) or n (B).  With vector width V,
// blocks V*q .. V*q+V-1 share 32 V consecutive lines and lane lr of block V*q + v takes
// line 32 V q + V lr + v: a lane's V lines are adjacent, so an operand stored along m or
// n gives it one V-float LDS read per k for V blocks (V = 1: line 32 f + lr).
template <int V>
__device__ __forceinline__ constexpr int frag_line(int f, int lr) {
  return 32 * V * (f / V) + V * lr + f % V;
}
constexpr int frag_vec(bool along_k, int F) { return along_k ? 1 : F % 4 == 0 ? 4 : F % 2 == 0 ? 2 : 1; }

// The fragments of k-group g of a wavefront's F blocks, whose lines start at w0:
// out[f][e] = X(w0 + frag_line<V>(f, lr), 16g + 8lh + e)
template <typename Op, int F, int V>
__device__ __forceinline__ void read_frags(const float* stage, int w0, int g, int lr, int lh, float (&out)[F][8]) {
  if constexpr (V == 1) {
#pragma unroll
    for (int f = 0; f < F; ++f) Op::read(stage, w0 + 32 * f + lr, g, lh, out[f]);
  } else {
#pragma unroll
    for (int q = 0; q < F / V; ++q) Op::template read_vec<V>(stage, w0 + 32 * V * q + V * lr, g, lh, V * q, out);
  }
}

// PACKED: the operands stored along m or n take Operand's packed layout (LDS-DMA loads).
template <int BM, int BN, int BK, int WM, int WN, int KS, bool TA, bool TB, bool PACKED = false>
struct MfmaCfg {
  static constexpr int KG = BK / (16 * KS);  // 16-deep k-groups per wavefront per K-tile
  static constexpr int kThreads = WM * WN * KS * 64;
  static constexpr int FM = BM / WM / 32, FN = BN / WN / 32;  // 32x32 blocks per wavefront
  using OpA = Operand<BM, BK, kThreads, !TA, PACKED && TA>;
  using OpB = Operand<BN, BK, kThreads, TB, PACKED && !TB>;
  // fragment vector widths (frag_line) of A along m and B along n
  static constexpr int VA = frag_vec(!TA, FM), VB = frag_vec(TB, FN);
  // LDS fragment-read instructions of one wavefront per 16-deep k-group
  static constexpr int kFragReads = (TA ? 8 * FM / VA : 2 * FM) + (TB ? 2 * FN : 8 * FN / VB);
  static constexpr int kStageFloats = OpA::kStageFloats + OpB::kStageFloats;
  static constexpr int kReduceFloats = KS > 1 ? KS * BM * BN : 0;
  static constexpr int kLdsFloats = 2 * kStageFloats > kReduceFloats ? 2 * kStageFloats : kReduceFloats;
  static_assert(FM >= 1 && FN >= 1, "wavefront tile at least 32 x 32");
  static_assert(KG >= 1 && KG * 16 * KS == BK, "K-tile split into 16-deep k-groups");
};

}  // namespace mfma_detail
}  // namespace sgemm_impl
