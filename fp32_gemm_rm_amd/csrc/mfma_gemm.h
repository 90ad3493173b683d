// SGEMM on the FP32 matrix cores of gfx950 (v_mfma_f32_32x32x2_f32): device code and
// launch templates, instantiated per operand orientation by k_mfma_{nn,nt,tn,tt}.hip.
//
// The pages' fastest designs are register-blocked tiles fed from padded,
// double-buffered shared memory (sgemmNN page; mhpn.cn "GEMM advanced" page
// sections 2-3) and, for half precision only, warp-level matrix fragments
// ("GPU-accelerated matrix computation ..." section 2.2).  On gfx950 the dense
// FP32 contraction belongs on the matrix cores, which take float32 operands
// directly, so this kernel keeps the pages' tiling and double buffering and
// replaces the per-thread FMA block with 32 x 32 x 2 MFMA tiles.
//
// MFMA operand layout (32x32x2, checked on the device with one-hot operands):
// lane l supplies A(l%32, kk = l/32) and B(kk = l/32, l%32); accumulator
// register i of lane l holds D(8*(i/4) + 4*(l/32) + i%4, l%32).  The sum over
// k may visit k in any order, so lane half h = l/32 of MFMA step e takes
// k = 8h + e of the 16-wide K-tile (e = 0..7): a lane then reads its eight A
// values as two contiguous 128-bit LDS loads.
//
// Workgroup: WM x WN x KS wavefronts.  WM x WN of them tile the BM x BN block
// of C (each owning (BM/WM) x (BN/WN) as 32 x 32 accumulators of 16 registers);
// KS of them share each such block and split every K-tile of BK = 16*KS*KG
// between them (KG 16-deep k-groups each).  Their partial sums are added through
// LDS in the fixed order ks = 0, 1, ..., KS-1, so results are deterministic; each
// of the KS wavefronts then finishes 1/KS of the block (sum, alpha/beta, store).
// KS > 1 lets small problems, whose output alone would give each
// SIMD a single wavefront, run 4 wavefronts per SIMD and hide LDS, barrier and
// MFMA latencies.
//
// Pipelines (one barrier per K-tile, two LDS stages):
//   mfma_tile (32 configuration): the global loads of tile t+2 are issued as tile t's
//     MFMAs start, into the second of two register sets, and tile t+1's registers are
//     stored half-way through those MFMAs; fragments are read from LDS at the start of
//     each k-group.
//   mfma_tile_pf (256, 192, 128 and 64 configurations, one 16-deep k-group per wavefront
//     and K-tile): fragments are read one K-tile ahead into a second register set, so no
//     MFMA waits for LDS; the global loads (one or two K-tiles ahead of their LDS
//     stores), LDS stores and fragment reads are interleaved with the MFMAs.
// LDS layout:
//   A tile, BM rows of BK floats (BK/4 16-byte chunks), no padding.  For
//     BK = 16, chunk c of row r is stored at chunk position c ^ ((r/4) % 4).  On
//     gfx950 a 128-bit LDS access serves 16 lanes per cycle from 64 banks of 4
//     bytes (16 chunk slots): the 16 lanes of a fragment read cover rows
//     r..r+15 at one logical chunk, and the 16 lanes of a tile store cover rows
//     r..r+3 (r a multiple of 4) at chunks 0..3; the XOR spreads both over 16
//     distinct chunk slots.  (With +4-word padding instead, the reads are
//     conflict-free but the stores are not.)
//   B tile, BK rows of BN floats with stride BN + 4 words, stored as loaded.
//     A fragment read is one word per lane: each half-wavefront reads 32
//     consecutive words of one row.
//   Transposed operands swap layouts: an operand whose rows run along k in
//   global memory (A, or B^T stored N x K) takes the swizzled k-contiguous form
//   and 128-bit fragment reads; one whose rows run along m or n (A^T stored
//   K x M, or B) takes the k-major padded form and 32-bit fragment reads.
// Tile order: the hardware hands workgroups to the 8 XCDs round robin; block
// ids are remapped so that each XCD works on a contiguous run of tiles, and
// the run walks GROUP_M tile-rows at a time, so the A and B panels of the
// tiles in flight on one XCD share its L2.
//
// Partial tiles.  In the 192, 128, 64 and 32 configurations the tile grid covers the whole
// matrix and the tiles that reach past M or N are guarded MFMA tiles, dispatched on
// which side they cross (past M, past N, or both), so that a tile past M only loads B
// as a full tile does.  In the 256 configuration the MFMA tiles cover [0, Mf) x [0, Nf)
// with Mf, Nf the largest multiples of 256, and the strips past them (columns [Nf, N)
// of rows [0, Mf), then rows [Mf, M) in full) are cut into 32 x 32 tiles computed by
// the bounds-checked register-blocked VALU tile (regblock_tile.h, 256 threads, 2 x 2
// outputs each): the scalar edge-tile path.  One edge tile per workgroup; its NT/256
// groups of 256 threads split the tile's K range (all groups run the same number of
// K-steps, so their barriers match) and add their partial sums through LDS in the
// fixed group order.  Edge workgroups take the highest block ids of the same launch.
// Ragged K is handled inside every MFMA tile: its last K-tile loads zeros past K.
//
// Stream-K (256 x 256 tiles, batch 1, with a caller workspace): when the full tiles do
// not fill whole waves of 256 workgroups, the last partial wave and the full wave before
// it are not run one tile per workgroup; their K-tiles, taken tile by tile, are cut into
// 256 equal contiguous ranges, one per workgroup (after "Stream-K" work decomposition;
// the pages' kernels all run one tile per thread block).  Pieces of a tile that fall in
// different ranges go to the workspace and a fix-up kernel adds them in range order,
// so the result is deterministic (its summation order differs from the one-tile path).
#pragma once

#include <type_traits>

#include "regblock_tile.h"

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
// with stride R + 4 and a fragment is eight 32-bit reads.
template <int R, int BK, int NT, bool KROWS>
struct Operand {
  static constexpr int KC = BK / 4;
  static constexpr int LOADS = R * BK / 4 / NT;  // float4 per thread per K-tile
  static constexpr int STRIDE = KROWS ? BK : R + 4;
  static constexpr int kStageFloats = KROWS ? R * BK : BK * (R + 4);
  static_assert(LOADS >= 1 && LOADS * NT * 4 == R * BK, "even load split");

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
      *reinterpret_cast<float4*>(stage + (KROWS ? swz_slot<BK>(row[i], col[i]) : row[i] * STRIDE + col[i])) =
          reg[SET][i];
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
      for (int e = 0; e < 8; ++e) out[e] = stage[(16 * g + 8 * lh + e) * STRIDE + rr];
    }
  }
};

template <int BM, int BN, int BK, int WM, int WN, int KS, bool TA, bool TB>
struct MfmaCfg {
  static constexpr int KG = BK / (16 * KS);  // 16-deep k-groups per wavefront per K-tile
  static constexpr int kThreads = WM * WN * KS * 64;
  static constexpr int FM = BM / WM / 32, FN = BN / WN / 32;  // 32x32 blocks per wavefront
  using OpA = Operand<BM, BK, kThreads, !TA>;
  using OpB = Operand<BN, BK, kThreads, TB>;
  static constexpr int kStageFloats = OpA::kStageFloats + OpB::kStageFloats;
  static constexpr int kReduceFloats = KS > 1 ? KS * BM * BN : 0;
  static constexpr int kLdsFloats = 2 * kStageFloats > kReduceFloats ? 2 * kStageFloats : kReduceFloats;
  static_assert(FM >= 1 && FN >= 1, "wavefront tile at least 32 x 32");
  static_assert(KG >= 1 && KG * 16 * KS == BK, "K-tile split into 16-deep k-groups");
};

// Where the tiles of one launch are: MFMA tiles first, then the edge tiles of the
// right strip, then those of the bottom strip.
struct TileMap {
  int tiles_m, tiles_n;    // MFMA tiles
  int Mf, Nf;              // extent they cover
  int right_m, right_n;    // 32 x 32 edge tiles in columns [Nf, N) of rows [0, Mf)
  int bottom_m, bottom_n;  // 32 x 32 edge tiles in rows [Mf, M)
  // stream-K (sk_wgs > 0): MFMA tiles [0, dp_tiles) run one per workgroup; the K-tiles of
  // tiles [dp_tiles, tiles_m * tiles_n) are split evenly over sk_wgs workgroups (see
  // StreamK); partial tiles go to ws
  int dp_tiles, sk_wgs;
  float* ws;
};

// The stream-K split: the K-tiles ("iterations") of the stream-K tiles, tile-major, are
// cut into sk_wgs equal contiguous ranges; range g is [start(g), start(g + 1)) with
// start(g) = floor(g * W / G) for W iterations over G workgroups.  A workgroup writes a
// tile that its range covers whole straight to C.  The pieces of a tile split between
// ranges go to workspace slots: the first piece of range g to slot 2g, the last to slot
// 2g + 1 (both BM x BN floats), and a fix-up pass adds them in range order.
struct StreamK {
  long long work;  // W = stream-K tiles x iters
  int iters;       // K-tiles per tile
  int wgs;         // G
  __device__ __forceinline__ long long start(int g) const { return (long long)g * work / wgs; }
  // the range holding iteration j (the last range starting at or before j; ranges are
  // empty only when there are fewer iterations than workgroups)
  __device__ __forceinline__ int owner(long long j) const { return (int)(((j + 1) * wgs - 1) / work); }
};

// C := alpha * x[u] + beta * C at the NV elements (row(u), col(u)) of this lane, given
// by coord(u, row, col); C is not read when beta == 0.  GUARD (bit 0: rows, bit 1:
// columns): elements past M or N are skipped.  Every C value of the batch is loaded before the first store: a load
// after a store into the same array would wait for that store (the compiler cannot tell
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

// K-tiles [kb, ke) of the BM x BN tile of C at (m0, n0).  part == nullptr: the range is
// the whole K range and the result goes to C (alpha, beta); otherwise the raw sums go to
// part, a BM x BN row-major block (a stream-K partial tile).  GUARD bit 0 (1): the tile
// reaches past M, bit 1 (2): past N (loads stay inside the matrix, stores skip what is
// past it).
template <int BM, int BN, int BK, int WM, int WN, int KS, bool TA, bool TB, bool VEC, int GUARD>
__device__ __forceinline__ void mfma_tile(const Problem& p, int m0, int n0, int kb, int ke, float* smem,
                                          float* part = nullptr) {
  using Cfg = MfmaCfg<BM, BN, BK, WM, WN, KS, TA, TB>;
  using OpA = typename Cfg::OpA;
  using OpB = typename Cfg::OpB;
  constexpr int FM = Cfg::FM, FN = Cfg::FN, KG = Cfg::KG;
  constexpr bool GA = (GUARD & 1) != 0, GB = (GUARD & 2) != 0;  // A rows past M, B columns past N
  // stage s: A at smem + s * kStageFloats, B right after it
  auto a_stage = [&](int s) { return smem + s * Cfg::kStageFloats; };
  auto b_stage = [&](int s) { return smem + s * Cfg::kStageFloats + OpA::kStageFloats; };

  const int t = threadIdx.x;
  const int w = t / 64, l = t % 64;
  const int lr = l % 32, lh = l / 32;
  // K-group and spatial position of this wavefront (compile-time zero K-group without a
  // K split, which keeps the fragment-read addresses foldable)
  const int ks = KS == 1 ? 0 : w / (WM * WN), sp = KS == 1 ? w : w % (WM * WN);
  const int wm0 = (sp / WN) * (BM / WM), wn0 = (sp % WN) * (BN / WN);

  OpA opa;
  OpB opb;
  opa.init(p.A, p.lda, m0, p.M - m0, t);
  opb.init(p.B, p.ldb, n0, p.N - n0, t);

  v16f acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nfull = p.K / BK;  // K-tiles with no element past K
  // global -> registers (set SET) for K-tile kt; the guarded form (the last, partial
  // K-tile only) loads zeros past K and is kept out of the steady-state loop
  auto load = [&](auto set, int kt) {
    constexpr int SET = decltype(set)::value;
    if (kt < nfull) {
      opa.template load_full<VEC, GA, SET>(kt * BK);
      opb.template load_full<VEC, GB, SET>(kt * BK);
    } else {
      opa.template load_tail<VEC, GA, SET>(kt * BK, p.K - kt * BK);
      opb.template load_tail<VEC, GB, SET>(kt * BK, p.K - kt * BK);
    }
  };
  // the MFMAs of K-tile kt from stage s; `mid` runs half-way through the last k-group
  auto multiply = [&](int s, auto mid) {
#pragma unroll
    for (int r = 0; r < KG; ++r) {
      const int g = ks * KG + r;  // 16-deep k-group of this K-tile
      float af[FM][8], bf[FN][8];
#pragma unroll
      for (int i = 0; i < FM; ++i) OpA::read(a_stage(s), wm0 + i * 32 + lr, g, lh, af[i]);
#pragma unroll
      for (int j = 0; j < FN; ++j) OpB::read(b_stage(s), wn0 + j * 32 + lr, g, lh, bf[j]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[i][e], bf[j][e], acc[i][j], 0, 0, 0);
        // store the next tile's registers into the other stage half-way through the last
        // k-group's MFMAs (that stage was last read before the previous barrier), so that
        // the LDS writes overlap MFMAs instead of bunching up before the barrier: +1.5%
        if (e == 3 && r == KG - 1) mid();
      }
    }
  };
  using Set0 = std::integral_constant<int, 0>;
  using Set1 = std::integral_constant<int, 1>;
  // Prefetch distance two: tile j's registers are set j % 2; tile kt+2 is loaded while
  // tile kt is multiplied and tile kt+1 (loaded one step earlier) is stored to LDS, so
  // each load has two K-tiles of MFMAs to arrive (one K-tile ahead is 2-10% slower;
  // 4096^3: 141.0 against 143.7 TFLOP/s).  The steady-state loop issues the same loads
  // and stores on every path, so that the compiler's wait before the LDS store covers
  // only the older register set (a wait on the newest loads would undo the prefetch);
  // the last steps run the general form.
  load(Set0{}, kb);
  opa.template store<0>(a_stage(0));
  opb.template store<0>(b_stage(0));
  if (kb + 1 < ke) load(Set1{}, kb + 1);
  __syncthreads();
  auto steady = [&](auto set, int kt) {  // set = (kt - kb) % 2, also the LDS stage of tile kt
    constexpr int P = decltype(set)::value;
    opa.template load_full<VEC, GA, P>((kt + 2) * BK);
    opb.template load_full<VEC, GB, P>((kt + 2) * BK);
    __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of the MFMAs
    multiply(P, [&] {
      opa.template store<P ^ 1>(a_stage(P ^ 1));
      opb.template store<P ^ 1>(b_stage(P ^ 1));
    });
    __syncthreads();
  };
  auto step = [&](auto set, int kt) {
    constexpr int P = decltype(set)::value;
    if (kt + 2 < ke) load(set, kt + 2);
    multiply(P, [&] {
      if (kt + 1 < ke) {
        opa.template store<P ^ 1>(a_stage(P ^ 1));
        opb.template store<P ^ 1>(b_stage(P ^ 1));
      }
    });
    __syncthreads();
  };
  int kt = kb;
  const int steady_end = min(ke, nfull);
  for (; kt + 3 < steady_end; kt += 2) {  // tiles kt+2 and kt+3 are full and in range
    steady(Set0{}, kt);
    steady(Set1{}, kt + 1);
  }
  for (; kt < ke; kt += 2) {
    step(Set0{}, kt);
    if (kt + 1 < ke) step(Set1{}, kt + 1);
  }

  finish_acc<BM, BN, WM, WN, KS, FM, FN, GUARD>(p, acc, smem, m0, n0, part);
}

// Scheduling groups for one K-tile of mfma_tile_pf: each of its NM MFMAs is followed by
// PER of its T memory instructions, in the order NW LDS writes, NL global loads, then
// the LDS fragment reads (sched_group_barrier masks 0x008 MFMA, 0x200 LDS write, 0x020
// global load, 0x100 LDS read).
template <int O, int E, int NW, int NL>
__device__ __forceinline__ void sched_mem_ops() {
  if constexpr (O < E) {
    __builtin_amdgcn_sched_group_barrier(O < NW ? 0x200 : O < NW + NL ? 0x020 : 0x100, 1, 0);
    sched_mem_ops<O + 1, E, NW, NL>();
  }
}
template <int I, int NM, int PER, int T, int NW, int NL>
__device__ __forceinline__ void sched_interleave() {
  if constexpr (I < NM && I * PER < T) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    sched_mem_ops<I * PER, (I * PER + PER < T ? I * PER + PER : T), NW, NL>();
    sched_interleave<I + 1, NM, PER, T, NW, NL>();
  }
}

// K-tiles [kb, ke) of the BM x BN tile at (m0, n0), as mfma_tile, for configurations with
// one 16-deep k-group per wavefront and K-tile (BK = 16 KS).  The MFMA fragments are read
// from LDS one K-tile ahead into a second register set, so that no MFMA waits for an LDS
// read: with fragments read after the barrier, right before the MFMAs that use them, the
// wavefronts lose 3-6% of the matrix-core cycles to LDS latency (probe: 150-146 against
// 155 TFLOP/s with no LDS reads), and more where a K-tile holds few MFMAs.
//   During K-tile t (fragment set P = (t - kb) % 2, LDS stage P):
//     - the fragments of tile t+1 are read from stage P^1 into set P^1;
//     - the global registers of tile t+2 are stored to stage P, whose fragments were
//       read before the previous barrier;
//     - tile t+2+NSETS is loaded into global register set P % NSETS, the one just stored;
//     - the MFMAs of tile t run on set P;
//   and one barrier ends the K-tile.  A global load has NSETS K-tiles of MFMAs to
//   arrive: one in the 256 and 192 configurations (128 and 72 MFMAs per wavefront and
//   K-tile; the 256 configuration has no registers to spare, and a second set measured
//   no better in the 192 one), two in the 128 and 64 configurations (32 and 8).
template <int BM, int BN, int BK, int WM, int WN, int KS, int NSETS, bool TA, bool TB, bool VEC, int GUARD>
__device__ __forceinline__ void mfma_tile_pf(const Problem& p, int m0, int n0, int kb, int ke, float* smem,
                                             float* part = nullptr) {
  using Cfg = MfmaCfg<BM, BN, BK, WM, WN, KS, TA, TB>;
  using OpA = typename Cfg::OpA;
  using OpB = typename Cfg::OpB;
  constexpr int FM = Cfg::FM, FN = Cfg::FN;
  static_assert(Cfg::KG == 1, "one k-group per wavefront and K-tile");
  static_assert(NSETS == 1 || NSETS == 2, "global register sets");
  constexpr bool GA = (GUARD & 1) != 0, GB = (GUARD & 2) != 0;  // A rows past M, B columns past N
  auto a_stage = [&](int s) { return smem + s * Cfg::kStageFloats; };
  auto b_stage = [&](int s) { return smem + s * Cfg::kStageFloats + OpA::kStageFloats; };

  const int t = threadIdx.x;
  const int w = t / 64, l = t % 64;
  const int lr = l % 32, lh = l / 32;
  // K-group and spatial position of this wavefront (compile-time zero K-group without a
  // K split, which keeps the fragment-read addresses foldable)
  const int ks = KS == 1 ? 0 : w / (WM * WN), sp = KS == 1 ? w : w % (WM * WN);
  const int wm0 = (sp / WN) * (BM / WM), wn0 = (sp % WN) * (BN / WN);

  OpA opa;
  OpB opb;
  opa.init(p.A, p.lda, m0, p.M - m0, t);
  opb.init(p.B, p.ldb, n0, p.N - n0, t);

  v16f acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  float af[2][FM][8], bf[2][FN][8];

  const int nfull = p.K / BK;
  auto load = [&](auto set, int kt) {
    constexpr int R = decltype(set)::value % NSETS;
    if (kt < nfull) {
      opa.template load_full<VEC, GA, R>(kt * BK);
      opb.template load_full<VEC, GB, R>(kt * BK);
    } else {
      opa.template load_tail<VEC, GA, R>(kt * BK, p.K - kt * BK);
      opb.template load_tail<VEC, GB, R>(kt * BK, p.K - kt * BK);
    }
  };
  auto store = [&](auto set, int s) {
    constexpr int R = decltype(set)::value % NSETS;
    opa.template store<R>(a_stage(s));
    opb.template store<R>(b_stage(s));
  };
  auto frags = [&](auto set, int s) {
    constexpr int S = decltype(set)::value;
#pragma unroll
    for (int i = 0; i < FM; ++i) OpA::read(a_stage(s), wm0 + i * 32 + lr, ks, lh, af[S][i]);
#pragma unroll
    for (int j = 0; j < FN; ++j) OpB::read(b_stage(s), wn0 + j * 32 + lr, ks, lh, bf[S][j]);
  };
  auto mfmas = [&](auto set) {
    constexpr int S = decltype(set)::value;
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[S][i][e], bf[S][j][e], acc[i][j], 0, 0, 0);
  };
  using Set0 = std::integral_constant<int, 0>;
  using Set1 = std::integral_constant<int, 1>;
  constexpr int D = 2 + NSETS;  // load distance in K-tiles, counted from the tile being multiplied

  // prologue: stage 0 <- tile kb (read into fragment set 0), stage 1 <- tile kb+1, global
  // registers <- tiles kb+2 .. kb+D-1
  load(Set0{}, kb);
  if constexpr (NSETS == 2)
    if (kb + 1 < ke) load(Set1{}, kb + 1);
  store(Set0{}, 0);
  if constexpr (NSETS == 1) {
    if (kb + 1 < ke) load(Set1{}, kb + 1);
  } else {
    if (kb + 2 < ke) load(Set0{}, kb + 2);
  }
  __syncthreads();
  frags(Set0{}, 0);
  if (kb + 1 < ke) store(Set1{}, 1);
  if (kb + D - 1 < ke) load(std::integral_constant<int, D - 1>{}, kb + D - 1);
  __syncthreads();

  // Instruction order of a steady K-tile: the MFMAs start right after the barrier and
  // each of the first ones is followed by its share of the memory instructions (LDS
  // stores, then global loads, then fragment reads), so that the wavefronts issue their
  // memory traffic in the shadow of the MFMAs; nothing moves across the barrier (the
  // compiler would otherwise hoist the barrier, and its wait on the fragment reads, above
  // the MFMAs).
  constexpr int kStores = OpA::LOADS + OpB::LOADS;
  constexpr int kLoads = OpA::kLoadInstrs(VEC) + OpB::kLoadInstrs(VEC);
  constexpr int kFragReads = FM * (OpA::STRIDE == BK ? 2 : 8) + FN * (OpB::STRIDE == BK ? 2 : 8);
  constexpr int kMfmas = 8 * FM * FN, kMemOps = kStores + kLoads + kFragReads;
  constexpr int kPer = (kMemOps + kMfmas - 1) / kMfmas;
  auto steady = [&](auto set, int kt) {  // tiles kt+1 .. kt+D exist and kt+D is full
    constexpr int P = decltype(set)::value;
    __builtin_amdgcn_sched_barrier(0);
    store(set, P);
    opa.template load_full<VEC, GA, P % NSETS>((kt + D) * BK);
    opb.template load_full<VEC, GB, P % NSETS>((kt + D) * BK);
    frags(std::integral_constant<int, P ^ 1>{}, P ^ 1);
    mfmas(set);
    sched_interleave<0, kMfmas, kPer, kMemOps, kStores, kLoads>();
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
  };
  auto step = [&](auto set, int kt) {
    constexpr int P = decltype(set)::value;
    if (kt + 2 < ke) store(set, P);
    if (kt + D < ke) load(set, kt + D);
    if (kt + 1 < ke) frags(std::integral_constant<int, P ^ 1>{}, P ^ 1);
    mfmas(set);
    __syncthreads();
  };
  int kt = kb;
  const int steady_end = min(ke, nfull);
  for (; kt + D + 1 < steady_end; kt += 2) {  // tiles kt+D and kt+D+1 are full and in range
    steady(Set0{}, kt);
    steady(Set1{}, kt + 1);
  }
  for (; kt < ke; kt += 2) {
    step(Set0{}, kt);
    if (kt + 1 < ke) step(Set1{}, kt + 1);
  }

  finish_acc<BM, BN, WM, WN, KS, FM, FN, GUARD>(p, acc, smem, m0, n0, part);
}

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
// first + nlines); width < EDGE_MIN <= 16 and nlines <= 16.  A strip that thin would cost
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
  float* red = smem;  // [wavefront][register][lane]
#pragma unroll
  for (int r = 0; r < 4; ++r) red[(wv * 4 + r) * 64 + l] = acc[r];
  __syncthreads();
  if (t < 256) {
    const int i = t / 16, j = t % 16, lane = 16 * (i / 4) + j, r = i % 4;
    const int line = cols ? i : j, out = cols ? j : i;
    if (line < nlines && out < width) {
      float x = red[r * 64 + lane];
#pragma unroll
      for (int q = 1; q < W; ++q) x += red[(q * 4 + r) * 64 + lane];
      const int row = cols ? first + line : lo + out, col = cols ? lo + out : first + line;
      float* c = p.C + (long long)row * p.ldc + col;
      *c = p.beta == 0.0f ? p.alpha * x : fmaf(p.alpha, x, p.beta * *c);
    }
  }
}

// Tile (bm, bn) of MFMA workgroup `bid`: XCD-contiguous, GROUP_M-row-major order.
template <int GROUP_M>
__device__ __forceinline__ void tile_coords(int bid, int tiles_m, int tiles_n, int& bm, int& bn) {
  const int nblk = tiles_m * tiles_n;
  if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
  const int group = GROUP_M * tiles_n;
  const int first_m = (bid / group) * GROUP_M;
  const int gsz = min(tiles_m - first_m, GROUP_M);
  bm = first_m + (bid % group) % gsz;
  bn = (bid % group) / gsz;
}

// MIN_BLOCKS workgroups must fit on one CU at once (a register budget for the compiler).
// EDGE_MIN: 0, the tiles cover [0, Mf) x [0, Nf) with Mf, Nf multiples of BM, BN and the
// strips past them are scalar edge tiles; otherwise a strip at least EDGE_MIN rows
// (columns) wide is covered by guarded MFMA tiles of the same grid and a thinner one runs
// as thin strips.  Edge tiles and thin strips take the block ids after the tiles (thin
// strips dispatched first measured slower: 1000 x 1030 x 999 24.8 -> 28.4 us).
// PF: the tiles run mfma_tile_pf (one k-group per wavefront and K-tile) instead of mfma_tile.
template <int BM, int BN, int BK, int WM, int WN, int KS, bool TA, bool TB, int GROUP_M, int MIN_BLOCKS,
          int EDGE_MIN, bool STREAM_K, bool VEC, bool PF>
__global__ __launch_bounds__(WM* WN* KS * 64) __attribute__((amdgpu_waves_per_eu(MIN_BLOCKS* WM* WN* KS / 4)))
void mfma_kernel(Problem p, TileMap map) {
  static_assert(!PF || BK == 16 * KS, "fragment prefetch: one 16-deep k-group per wavefront and K-tile");
  using Cfg = MfmaCfg<BM, BN, BK, WM, WN, KS, TA, TB>;
  p = batch_entry(p);
  constexpr int kGroups = Cfg::kThreads / 256;
  constexpr bool kEdges = EDGE_MIN == 0, kThin = EDGE_MIN > 1;  // scalar edge tiles / thin strips may exist
  static_assert(EDGE_MIN <= kThinMax, "thin strips are at most kThinMax wide");
  constexpr int kEdgeFloats = kEdges ? kGroups * EdgeTile::kLdsFloats  // >= its reduction floats
                                     : kThin ? Cfg::kThreads / 64 * 4 * 64 : 0;
  constexpr int kFloats = Cfg::kLdsFloats > kEdgeFloats ? Cfg::kLdsFloats : kEdgeFloats;
  static_assert(kFloats * 4 <= 160 * 1024, "LDS of one workgroup fits a CU");
  __shared__ __attribute__((aligned(16))) float smem[kFloats];
  // the MFMA tiles see the matrix as [0, Mf) x [0, Nf): what lies past it is the strips'
  Problem pt = p;
  pt.M = map.Mf;
  pt.N = map.Nf;
  auto tile = [&](auto guard, int m0, int n0, int kb, int ke, float* part) {
    constexpr int G = decltype(guard)::value;
    if constexpr (PF)
      mfma_tile_pf<BM, BN, BK, WM, WN, KS, (BM >= 192 ? 1 : 2), TA, TB, VEC, G>(pt, m0, n0, kb, ke, smem, part);
    else
      mfma_tile<BM, BN, BK, WM, WN, KS, TA, TB, VEC, G>(pt, m0, n0, kb, ke, smem, part);
  };
  const int nmfma = map.tiles_m * map.tiles_n;
  const int ndp = STREAM_K ? map.dp_tiles : nmfma;
  const int iters = (p.K + BK - 1) / BK;
  int e = (int)blockIdx.x - ndp;
  if (e < 0) {  // one whole tile
    int bm, bn;
    tile_coords<GROUP_M>(blockIdx.x, map.tiles_m, map.tiles_n, bm, bn);
    const int m0 = bm * BM, n0 = bn * BN;
    const bool past_m = EDGE_MIN != 0 && m0 + BM > pt.M, past_n = EDGE_MIN != 0 && n0 + BN > pt.N;
    if (!past_m && !past_n)
      tile(std::integral_constant<int, 0>{}, m0, n0, 0, iters, nullptr);
    else if (!past_n)
      tile(std::integral_constant<int, 1>{}, m0, n0, 0, iters, nullptr);
    else if (!past_m)
      tile(std::integral_constant<int, 2>{}, m0, n0, 0, iters, nullptr);
    else
      tile(std::integral_constant<int, 3>{}, m0, n0, 0, iters, nullptr);
    return;
  }
  if (STREAM_K && e < map.sk_wgs) {  // one stream-K range (full tiles only)
    const StreamK sk{(long long)(nmfma - map.dp_tiles) * iters, iters, map.sk_wgs};
    const long long j0 = sk.start(e), j1 = sk.start(e + 1);
    for (long long j = j0; j < j1;) {
      const int u = (int)(j / iters);  // stream-K tile
      const long long tile_end = (long long)(u + 1) * iters;
      const long long seg_end = j1 < tile_end ? j1 : tile_end;
      const int kb = (int)(j - (long long)u * iters), ke = (int)(seg_end - (long long)u * iters);
      float* part = nullptr;
      if (kb > 0 || ke < iters)
        part = map.ws + (2LL * e + (j == j0 ? 0 : 1)) * (long long)(BM * BN);
      int bm, bn;
      tile_coords<GROUP_M>(map.dp_tiles + u, map.tiles_m, map.tiles_n, bm, bn);
      if (j != j0) __syncthreads();  // the previous piece's epilogue may still read LDS
      tile(std::integral_constant<int, 0>{}, bm * BM, bn * BN, kb, ke, part);
      j = seg_end;
    }
    return;
  }
  if (STREAM_K) e -= map.sk_wgs;
  if constexpr (kEdges) {
    int m0, n0;
    const int n_right = map.right_m * map.right_n;
    if (e < n_right) {
      m0 = (e / map.right_n) * kEdge;
      n0 = map.Nf + (e % map.right_n) * kEdge;
    } else {
      e -= n_right;
      m0 = map.Mf + (e / map.bottom_n) * kEdge;
      n0 = (e % map.bottom_n) * kEdge;
    }
    edge_tile<kGroups, TA, TB, VEC>(p, m0, n0, smem);
  }
  if constexpr (kThin) {
    const int n_right = map.right_m;  // right strip: columns [Nf, N) of rows [0, Mf)
    if (e < n_right) {
      const int first = e * kThinMax;
      thin_strip<Cfg::kThreads, TA, TB, VEC>(p, true, first, min(kThinMax, map.Mf - first), map.Nf, p.N - map.Nf, smem);
    } else {  // bottom strip: rows [Mf, M) of columns [0, N)
      const int first = (e - n_right) * kThinMax;
      thin_strip<Cfg::kThreads, TA, TB, VEC>(p, false, first, min(kThinMax, p.N - first), map.Mf, p.M - map.Mf, smem);
    }
  }
}

// Stream-K fix-up: kFixSlices workgroups per stream-K tile that was split between ranges,
// each over BM / kFixSlices rows; adds the pieces in range order and applies alpha and
// beta.  Tiles that one range covered whole were written by the main kernel.  Each thread
// takes kFixQuads float4s of the slice and issues all of their loads (every piece, then
// C) before its first store, so that the memory-bound pass keeps many loads in flight
// (one workgroup per tile, each thread walking its float4s one by one, took 87 us for
// 272 tiles at 4352 x 4096).
constexpr int kFixSlices = 8;
template <int BM, int BN, int BK, int GROUP_M>
__global__ __launch_bounds__(256) void sk_fixup_kernel(Problem p, TileMap map) {
  constexpr int kQuads = BN / 4;                         // float4 per row
  constexpr int kSliceQuads = BM / kFixSlices * kQuads;  // float4 per slice
  constexpr int kFixQuads = kSliceQuads / 256;           // float4 per thread
  static_assert(kFixQuads * 256 == kSliceQuads, "even split of a slice over 256 threads");
  const int nmfma = map.tiles_m * map.tiles_n;
  const int iters = (p.K + BK - 1) / BK;
  const StreamK sk{(long long)(nmfma - map.dp_tiles) * iters, iters, map.sk_wgs};
  const int u = blockIdx.x;
  const int g0 = sk.owner((long long)u * iters), g1 = sk.owner((long long)(u + 1) * iters - 1);
  if (g0 == g1) return;
  int bm, bn;
  tile_coords<GROUP_M>(map.dp_tiles + u, map.tiles_m, map.tiles_n, bm, bn);
  const int m0 = bm * BM, n0 = bn * BN, r0 = blockIdx.y * (BM / kFixSlices);
  float4 sum[kFixQuads];
  bool first = true;
  for (int g = g0; g <= g1; ++g) {
    if (sk.start(g) == sk.start(g + 1)) continue;  // empty range (fewer iterations than workgroups)
    const long long slot = 2LL * g + (sk.start(g) / iters == u ? 0 : 1);
    const float* piece = map.ws + slot * (BM * BN) + r0 * BN;
#pragma unroll
    for (int i = 0; i < kFixQuads; ++i) {
      const float4 v = *reinterpret_cast<const float4*>(piece + 4 * (threadIdx.x + 256 * i));
      if (first) {
        sum[i] = v;
      } else {
        sum[i].x += v.x; sum[i].y += v.y; sum[i].z += v.z; sum[i].w += v.w;
      }
    }
    first = false;
  }
  const bool vec_c = reinterpret_cast<uintptr_t>(p.C) % 16 == 0 && p.ldc % 4 == 0;
  auto crow = [&](int i) {
    const int q = threadIdx.x + 256 * i;
    return p.C + (long long)(m0 + r0 + q / kQuads) * p.ldc + n0 + (q % kQuads) * 4;
  };
  float4 c[kFixQuads];
  if (p.beta != 0.0f) {
#pragma unroll
    for (int i = 0; i < kFixQuads; ++i) {
      const float* q = crow(i);
      c[i] = vec_c ? *reinterpret_cast<const float4*>(q) : make_float4(q[0], q[1], q[2], q[3]);
    }
  }
#pragma unroll
  for (int i = 0; i < kFixQuads; ++i) {
    float4 o;
    if (p.beta == 0.0f) {
      o = make_float4(p.alpha * sum[i].x, p.alpha * sum[i].y, p.alpha * sum[i].z, p.alpha * sum[i].w);
    } else {
      o = make_float4(fmaf(p.alpha, sum[i].x, p.beta * c[i].x), fmaf(p.alpha, sum[i].y, p.beta * c[i].y),
                      fmaf(p.alpha, sum[i].z, p.beta * c[i].z), fmaf(p.alpha, sum[i].w, p.beta * c[i].w));
    }
    float* q = crow(i);
    if (vec_c) {
      *reinterpret_cast<float4*>(q) = o;
    } else {
      q[0] = o.x; q[1] = o.y; q[2] = o.z; q[3] = o.w;
    }
  }
}

// ws != nullptr (batch 1, configurations with EDGE_MIN = 0): stream-K over 256
// workgroups for the last partial wave of tiles plus one full wave before it (the tiles
// before those run one per workgroup); ws holds 2 * 256 * BM * BN floats.
template <int BM, int BN, int BK, int WM, int WN, int KS, bool TA, bool TB, int GROUP_M, int MIN_BLOCKS,
          int EDGE_MIN = 0, bool PF = false>
hipError_t launch_cfg(const Problem& p, int batch, hipStream_t stream, float* ws = nullptr) {
  static_assert(BM == BN && BM % kEdge == 0, "square tiles whose sides are multiples of the edge tile");
  TileMap map;
  map.dp_tiles = map.sk_wgs = 0;
  map.ws = nullptr;
  // extent of the MFMA tiles: rows [0, Mf), columns [0, Nf) (mfma_extent, tile_plan.h uses
  // the same rule); the strips past it (columns [Nf, N) of rows [0, Mf), then rows [Mf, M)
  // of every column) are scalar edge tiles or thin strips
  map.Mf = mfma_extent(p.M, BM, EDGE_MIN);
  map.Nf = mfma_extent(p.N, BN, EDGE_MIN);
  if constexpr (EDGE_MIN > 1) {
    // Guarded tiles load an operand stored along m or n (A^T, B) in whole float4s, so its
    // limit must be a multiple of 4: the last 1-3 rows (columns) join the thin strips (the
    // tile count does not change: a guarded remainder is at least 4 wide).
    if (TA) map.Mf &= ~3;
    if (!TB) map.Nf &= ~3;
  }
  map.tiles_m = (map.Mf + BM - 1) / BM;
  map.tiles_n = (map.Nf + BN - 1) / BN;
  if (map.tiles_m == 0 || map.tiles_n == 0) {  // no MFMA tile
    map.tiles_m = map.tiles_n = 0;
    // scalar edge tiles: everything is the bottom strip; thin strips: M or N is thinner
    // than EDGE_MIN and the strips as defined cover the matrix
    if (EDGE_MIN <= 1) map.Mf = map.Nf = 0;
  }
  if constexpr (EDGE_MIN > 1) {  // thin strips, in workgroups of kThinMax lines
    map.right_m = (map.Nf < p.N) ? (map.Mf + kThinMax - 1) / kThinMax : 0;
    map.right_n = map.right_m > 0 ? 1 : 0;
    map.bottom_n = (map.Mf < p.M) ? (p.N + kThinMax - 1) / kThinMax : 0;
    map.bottom_m = map.bottom_n > 0 ? 1 : 0;
  } else {
    map.right_m = (map.Nf < p.N) ? (map.Mf + kEdge - 1) / kEdge : 0;
    map.right_n = (map.Nf < p.N) ? (p.N - map.Nf + kEdge - 1) / kEdge : 0;
    map.bottom_m = (p.M - map.Mf + kEdge - 1) / kEdge;
    map.bottom_n = map.bottom_m > 0 ? (p.N + kEdge - 1) / kEdge : 0;
  }
  const long long nmfma = (long long)map.tiles_m * map.tiles_n;
  const long long edge_tiles = (long long)map.right_m * map.right_n + (long long)map.bottom_m * map.bottom_n;
  const dim3 block(WM * WN * KS * 64);
  const bool vec = vec4_ok(p.A, p.lda) && vec4_ok(p.B, p.ldb);
  if constexpr (EDGE_MIN == 0 && BM == 256 && BN == 256) {  // the workspace holds 256 x 256 slots
    if (ws != nullptr && batch == 1 && nmfma % kStreamKWgs != 0) {
      const long long sk_tiles = nmfma % kStreamKWgs + (nmfma > kStreamKWgs ? kStreamKWgs : 0);
      map.dp_tiles = (int)(nmfma - sk_tiles);
      map.sk_wgs = kStreamKWgs;
      map.ws = ws;
      const long long blocks = map.dp_tiles + map.sk_wgs + edge_tiles;
      if (blocks > kMaxGrid) return hipErrorInvalidConfiguration;
      if (vec)
        hipLaunchKernelGGL((mfma_kernel<BM, BN, BK, WM, WN, KS, TA, TB, GROUP_M, MIN_BLOCKS, 0, true, true, PF>),
                           dim3((unsigned)blocks), block, 0, stream, p, map);
      else
        hipLaunchKernelGGL((mfma_kernel<BM, BN, BK, WM, WN, KS, TA, TB, GROUP_M, MIN_BLOCKS, 0, true, false, PF>),
                           dim3((unsigned)blocks), block, 0, stream, p, map);
      const hipError_t err = hipGetLastError();
      if (err != hipSuccess) return err;
      hipLaunchKernelGGL((sk_fixup_kernel<BM, BN, BK, GROUP_M>), dim3((unsigned)sk_tiles, kFixSlices), dim3(256), 0,
                         stream, p, map);
      return hipGetLastError();
    }
  }
  const long long blocks = nmfma + edge_tiles;
  if (blocks > kMaxGrid) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)blocks, batch);
  if (vec)
    hipLaunchKernelGGL((mfma_kernel<BM, BN, BK, WM, WN, KS, TA, TB, GROUP_M, MIN_BLOCKS, EDGE_MIN, false, true, PF>),
                       grid, block, 0, stream, p, map);
  else
    hipLaunchKernelGGL((mfma_kernel<BM, BN, BK, WM, WN, KS, TA, TB, GROUP_M, MIN_BLOCKS, EDGE_MIN, false, false, PF>),
                       grid, block, 0, stream, p, map);
  return hipGetLastError();
}

// The tile configurations (tile_plan.h), by tile side.  All but the 32 configuration run
// mfma_tile_pf (fragments read one K-tile ahead).
//   256: 256 x 256 tiles, 2 x 2 wavefronts of 128 x 128 (one per SIMD, 256 accumulator
//        registers each), BK 16, one global register set: one workgroup per CU.
//   192: 192 x 192 tiles, 2 x 2 wavefronts of 96 x 96 (144 accumulator registers), BK 16,
//        one global register set: one workgroup per CU.  Its tile counts fill whole waves
//        where the others do not (3072^3: 256 tiles).
//   128: 128 x 128 tiles, 2 x 2 wavefronts of 64 x 64, BK 16, two global register sets;
//        two workgroups per CU (three spill registers).
//   64:  64 x 64 tiles, 2 x 2 wavefronts of 32 x 32 and a 2-way K split, BK 32, two
//        global register sets; two workgroups per CU.
//   32:  32 x 32 tiles, one 32 x 32 block per wavefront and a 4-way K split, BK 64,
//        256 threads, mfma_tile; four workgroups per CU.
// Partial tiles (mfma_edge_min): guarded MFMA tiles of the same grid in the 192, 128, 64
// and 32 configurations, except strips thinner than 16 in the 192, 128 and 64
// configurations (thin strips); the scalar edge-tile path in the 256 configuration.
// ws: stream-K workspace (kStreamKBytes) for the 256 configuration, or nullptr.
template <bool TA, bool TB>
hipError_t launch_op(const Problem& p, int batch, hipStream_t stream, int tiles, float* ws = nullptr) {
  switch (tiles) {
    case 256:
      return launch_cfg<256, 256, 16, 2, 2, 1, TA, TB, 8, 1, mfma_edge_min(256), true>(p, batch, stream, ws);
    case 192:
      if (p.M % 192 == 0 && p.N % 192 == 0)
        return launch_cfg<192, 192, 16, 2, 2, 1, TA, TB, 8, 1, 0, true>(p, batch, stream);
      return launch_cfg<192, 192, 16, 2, 2, 1, TA, TB, 8, 1, mfma_edge_min(192), true>(p, batch, stream);
    case 128:
      if (p.M % 128 == 0 && p.N % 128 == 0)
        return launch_cfg<128, 128, 16, 2, 2, 1, TA, TB, 8, 2, 0, true>(p, batch, stream);
      return launch_cfg<128, 128, 16, 2, 2, 1, TA, TB, 8, 2, mfma_edge_min(128), true>(p, batch, stream);
    case 64:
      if (p.M % 64 == 0 && p.N % 64 == 0) return launch_cfg<64, 64, 32, 2, 2, 2, TA, TB, 8, 2, 0, true>(p, batch, stream);
      return launch_cfg<64, 64, 32, 2, 2, 2, TA, TB, 8, 2, mfma_edge_min(64), true>(p, batch, stream);
    case 32:
      if (p.M % 32 == 0 && p.N % 32 == 0) return launch_cfg<32, 32, 64, 1, 1, 4, TA, TB, 8, 4>(p, batch, stream);
      return launch_cfg<32, 32, 64, 1, 1, 4, TA, TB, 8, 4, mfma_edge_min(32)>(p, batch, stream);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace mfma_detail
}  // namespace sgemm_impl
