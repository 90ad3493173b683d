// SGEMM on the FP32 matrix cores of gfx950 (v_mfma_f32_32x32x2_f32): device code and
// launch templates, instantiated per operand orientation by k_mfma_{nn,nt,tn,tt}.hip.
// This file holds the overview below, the launch map, the kernels and their launch; the
// parts live in mfma_operand.h (LDS layouts, loads, fragments), mfma_tiles.h (the K-loop
// pipelines), mfma_epilogue.h (C updates, K-split reduction) and mfma_strips.h (edge tiles
// and thin strips).
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
// Pipelines (one barrier per K-tile):
//   mfma_tile (32 configuration): the global loads of tile t+2 are issued as tile t's
//     MFMAs start, into the second of two register sets, and tile t+1's registers are
//     stored half-way through those MFMAs; fragments are read from LDS at the start of
//     each k-group.
//   mfma_tile_pf (256, 192, 128 and 64 configurations, one 16-deep k-group per wavefront
//     and K-tile): fragments are read one K-tile ahead into a second register set, so
//     no MFMA waits for LDS; the global loads (one K-tile ahead of their LDS stores in
//     the 192 configuration, two in the others), LDS stores and fragment reads are
//     interleaved with the MFMAs.  Two LDS stages.
//   mfma_tile_direct (256, 192, 128 and 64 configurations with 16-byte aligned rows,
//     mfma_direct.h): as mfma_tile_pf, but the operands go from global memory straight
//     to LDS (LDS-DMA loads, four stages, issued four K-tiles ahead): no register
//     staging, no LDS stores, and with the registers this frees, two wavefronts per SIMD
//     in the 256 configuration.  Below 256 the operands stored along m or n take a packed
//     B layout (stride BN, columns XOR 32 in k-rows 8-15 of every 16), so that one 1 KiB
//     load fills whole k-rows.
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
// not fill whole waves of 256 workgroups, the last partial wave (and the full wave before
// it, where the partial one holds fewer than 32 tiles) is not run one tile per workgroup;
// its K-tiles, taken tile by tile, are cut into
// 256 equal contiguous ranges, one per workgroup (after "Stream-K" work decomposition;
// the pages' kernels all run one tile per thread block).  Pieces of a tile that fall in
// different ranges go to the workspace and a fix-up kernel adds them in range order,
// so the result is deterministic (its summation order differs from the one-tile path).
#pragma once

#include <type_traits>

#include "mfma_direct.h"
#include "mfma_strips.h"
#include "mfma_tiles.h"

namespace sgemm_impl {
namespace mfma_detail {

// Where the tiles of one launch are: MFMA tiles first, then the edge tiles (32 x 32) or
// thin strips (16 lines each) of the right strip, then those of the bottom strip.
struct TileMap {
  int tiles_m, tiles_n;    // MFMA tiles
  int Mf, Nf;              // extent they cover
  int right_m, right_n;    // edge tiles / thin strips in columns [Nf, N) of rows [0, Mf)
  int bottom_m, bottom_n;  // edge tiles / thin strips in rows [Mf, M)
  // stream-K (sk_wgs > 0): MFMA tiles [0, dp_tiles) run one per workgroup; the K-tiles of
  // tiles [dp_tiles, tiles_m * tiles_n) are split evenly over sk_wgs workgroups (see
  // StreamK); partial tiles go to ws
  int dp_tiles, sk_wgs;
  float* ws;
  // K slices (SLICED kernels, slices > 1): workgroup u + s * tiles computes the K-tiles
  // [s iters / slices, (s + 1) iters / slices) of tile u into workspace slot s * tiles + u
  int slices;
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
// FUSE: the right thin strip is computed inside the tiles (FusedStrip): tile (bm, bn) takes
// strip rows [bm BM + 4 bn, + 4), and the launch holds no right-strip workgroups.
// DIRECT (VEC, direct_ok): the tiles run mfma_tile_direct; 2: with its partial-last-K-tile
// path (the 64 configuration, K not a multiple of BK).
template <int BM, int BN, int BK, int WM, int WN, int KS, bool TA, bool TB, int GROUP_M, int MIN_BLOCKS,
          int EDGE_MIN, bool STREAM_K, bool VEC, bool PF, bool FUSE = false, bool SLICED = false,
          int DIRECT = 0>
__global__ __launch_bounds__(WM* WN* KS * 64) __attribute__((amdgpu_waves_per_eu(MIN_BLOCKS* WM* WN* KS / 4)))
void mfma_kernel(Problem p, TileMap map) {
  using Cfg = MfmaCfg<BM, BN, BK, WM, WN, KS, TA, TB>;
  p = batch_entry(p);
  constexpr int kGroups = Cfg::kThreads / 256;
  constexpr bool kEdges = EDGE_MIN == 0, kThin = EDGE_MIN > 1;  // scalar edge tiles / thin strips may exist
  // guarded MFMA tiles may exist (the register-staged 256 configuration's thin-strip form has
  // none: its launches have remainders thinner than kThin256 only; the direct one's guarded
  // form has both)
  constexpr bool kGuarded = EDGE_MIN != 0 && (BM != 256 || DIRECT);
  static_assert(BM != 256 || EDGE_MIN == 0 || EDGE_MIN == kThin256, "256 tiles: scalar edges or thin strips");
  static_assert(kThin256 == kThinMax, "the 256 thin-strip form's remainders fit one thin strip");
  static_assert(EDGE_MIN <= kThinMax, "thin strips are at most kThinMax wide");
  constexpr int kEdgeFloats = kEdges ? kGroups * EdgeTile::kLdsFloats  // >= its reduction floats
                                     : kThin ? thin_red_floats<Cfg::kThreads>() : 0;
  constexpr int kFuseFloats = FUSE ? 2 * Cfg::kStageFloats + 2 * FusedStrip<BK, Cfg::kThreads>::kStageFloats : 0;
  static_assert(!DIRECT || (BM == BN && VEC && !FUSE && !SLICED), "the direct pipeline: square tiles");
  constexpr int kDirectFloats = DIRECT ? kDirectStages * Cfg::kStageFloats : 0;
  constexpr int kFloats0 = Cfg::kLdsFloats > kEdgeFloats ? Cfg::kLdsFloats : kEdgeFloats;
  constexpr int kFloats1 = kFloats0 > kFuseFloats ? kFloats0 : kFuseFloats;
  constexpr int kFloats = kFloats1 > kDirectFloats ? kFloats1 : kDirectFloats;
  static_assert(kFloats * 4 <= 160 * 1024, "LDS of one workgroup fits a CU");
  __shared__ __attribute__((aligned(16))) float smem[kFloats];
  poison_lds(smem, kFloats);
  // the MFMA tiles see the matrix as [0, Mf) x [0, Nf): what lies past it is the strips'
  Problem pt = p;
  pt.M = map.Mf;
  pt.N = map.Nf;
  // fused strip rows of the tile being run (FUSE; set by the one-tile branch below)
  int srow0 = 0, srows = 0;
  // always inlined: called from the one-tile and the stream-K branches, the compiler would
  // otherwise emit it as a function, whose call spills the accumulators
  auto tile = [&](auto guard, int m0, int n0, int kb, int ke, float* part) __attribute__((always_inline)) {
    // guard bits 0-1 (the tile's partial sides), bit 2: the launch has full tiles only
    constexpr int G = decltype(guard)::value | (kGuarded ? 0 : 4);
    if constexpr (DIRECT)
      mfma_tile_direct<BM, BK, WM, WN, KS, TA, TB, G, DIRECT == 2>(pt, m0, n0, kb, ke, smem, part);
    else if constexpr (PF)
      mfma_tile_pf<BM, BN, BK, WM, WN, KS, (BM == 192 ? 1 : 2), TA, TB, VEC, G, FUSE>(
          pt, m0, n0, kb, ke, smem, part, srow0, srows, map.Nf, p.N - map.Nf);
    else
      mfma_tile<BM, BN, BK, WM, WN, KS, TA, TB, VEC, G>(pt, m0, n0, kb, ke, smem, part);
  };
  const int nmfma = map.tiles_m * map.tiles_n;
  const int ndp = STREAM_K ? map.dp_tiles : nmfma;
  const int iters = (p.K + BK - 1) / BK;
  // the guard form of tile (m0, n0): full, past M, past N or both
  auto guarded_tile = [&](int m0, int n0, int kb, int ke, float* part) __attribute__((always_inline)) {
    if constexpr (kGuarded) {
      const bool past_m = m0 + BM > pt.M, past_n = n0 + BN > pt.N;
      if (!past_m && !past_n)
        tile(std::integral_constant<int, 0>{}, m0, n0, kb, ke, part);
      else if (!past_n)
        tile(std::integral_constant<int, 1>{}, m0, n0, kb, ke, part);
      else if (!past_m)
        tile(std::integral_constant<int, 2>{}, m0, n0, kb, ke, part);
      else
        tile(std::integral_constant<int, 3>{}, m0, n0, kb, ke, part);
    } else {
      tile(std::integral_constant<int, 0>{}, m0, n0, kb, ke, part);
    }
  };
  if constexpr (SLICED) {  // one K slice of one tile, raw to the workspace (no strips in the launch)
    static_assert(!STREAM_K && !FUSE, "K slices run alone");
    const int u = (int)blockIdx.x % nmfma, s = (int)blockIdx.x / nmfma;
    int bm, bn;
    tile_coords<GROUP_M>(u, map.tiles_m, map.tiles_n, bm, bn);
    const int kb = (int)((long long)s * iters / map.slices), ke = (int)((long long)(s + 1) * iters / map.slices);
    guarded_tile(bm * BM, bn * BN, kb, ke, map.ws + ((long long)s * nmfma + u) * (BM * BN));
  } else {
    int e = (int)blockIdx.x - ndp;
    if (e < 0) {  // one whole tile
      int bm, bn;
      tile_coords<GROUP_M>(blockIdx.x, map.tiles_m, map.tiles_n, bm, bn);
      const int m0 = bm * BM, n0 = bn * BN;
      if constexpr (FUSE) {
        constexpr int SR = FusedStrip<BK, Cfg::kThreads>::SR;
        srow0 = m0 + SR * bn;
        srows = max(0, min(SR, min(m0 + BM, map.Mf) - srow0));
      }
      guarded_tile(m0, n0, 0, iters, nullptr);
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
        thin_strip<Cfg::kThreads, TA, TB, VEC>(p, true, first, min(kThinMax, map.Mf - first), map.Nf,
                                               p.N - map.Nf, smem);
      } else {  // bottom strip: rows [Mf, M) of columns [0, N)
        const int first = (e - n_right) * kThinMax;
        thin_strip<Cfg::kThreads, TA, TB, VEC>(p, false, first, min(kThinMax, p.N - first), map.Mf,
                                               p.M - map.Mf, smem);
      }
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

// K-slice fix-up: C := alpha * (sum of the tile's slices) + beta * C over the matrix part
// of the tiles, one workgroup per tile row (BN / 4 float4 columns, kSliceGroups groups of
// threads).  Group g adds slices [g S / G, (g + 1) S / G) in order (G = min(S,
// kSliceGroups)), and the groups' sums are added in group order through LDS: a fixed
// order, so results are deterministic, and no thread waits on a long chain of loads
// (a single thread per output over 256 slices would issue 256 dependent additions).
constexpr int kSliceGroups = 16;
template <int BM, int BN, int GROUP_M>
__global__ __launch_bounds__(BN / 4 * kSliceGroups) void slice_fixup_kernel(Problem p, TileMap map) {
  constexpr int kQuads = BN / 4;
  __shared__ float4 red[kSliceGroups][kQuads];
  poison_lds(&red[0][0].x, kSliceGroups * kQuads * 4);
  const int q = threadIdx.x % kQuads, g = threadIdx.x / kQuads;
  const int nmfma = map.tiles_m * map.tiles_n, u = blockIdx.x, r = blockIdx.y;
  const int S = map.slices, G = S < kSliceGroups ? S : kSliceGroups;
  float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
  if (g < G) {
    const int s0 = (int)((long long)g * S / G), s1 = (int)((long long)(g + 1) * S / G);
    const float* col = map.ws + (long long)u * (BM * BN) + r * BN + 4 * q;
    auto slice = [&](int s) { return *reinterpret_cast<const float4*>(col + (long long)s * nmfma * (BM * BN)); };
    auto add = [&](const float4& v) { sum.x += v.x; sum.y += v.y; sum.z += v.z; sum.w += v.w; };
    sum = slice(s0);
    int s = s0 + 1;
    for (; s + 4 <= s1; s += 4) {  // four loads in flight, added in slice order
      const float4 v0 = slice(s), v1 = slice(s + 1), v2 = slice(s + 2), v3 = slice(s + 3);
      add(v0);
      add(v1);
      add(v2);
      add(v3);
    }
    for (; s < s1; ++s) add(slice(s));
  }
  red[g][q] = sum;
  __syncthreads();
  if (g != 0) return;
  for (int h = 1; h < G; ++h) {
    const float4 v = red[h][q];
    sum.x += v.x; sum.y += v.y; sum.z += v.z; sum.w += v.w;
  }
  int bm, bn;
  tile_coords<GROUP_M>(u, map.tiles_m, map.tiles_n, bm, bn);
  const int row = bm * BM + r, col0 = bn * BN + 4 * q;
  if (row >= p.M) return;
  float* c = p.C + (long long)row * p.ldc + col0;
  const float x[4] = {sum.x, sum.y, sum.z, sum.w};
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (col0 + e < p.N) c[e] = p.beta == 0.0f ? p.alpha * x[e] : fmaf(p.alpha, x[e], p.beta * c[e]);
}

// ws != nullptr (batch 1, configurations with EDGE_MIN = 0): stream-K over 256
// workgroups for the last partial wave of tiles, plus the full wave before it where the
// partial one holds fewer than 32 tiles (the tiles before those run one per workgroup);
// ws holds 2 * 256 * BM * BN floats.  Measured, us, partial wave alone against with the
// wave before it: 5120^3 1911 / 1923, 4608^3 1423 / 1440, 6144^3 3227 / 3247,
// 5120 x 5120 x 2048 823 / 833; 4352 x 4096 x 4096 (16 tiles in the partial wave) 1095 / 1079.
//
// slices > 1 (ws != nullptr, batch 1, the 64 configuration, a launch of MFMA tiles only):
// every tile's K-tiles are cut into `slices` contiguous slices, each a workgroup that writes
// its raw partial tile to ws (slices x tiles x BM x BN floats), and slice_fixup_kernel adds
// them in slice order and applies alpha and beta.  For products of few tiles and long K.
template <int BM, int BN, int BK, int WM, int WN, int KS, bool TA, bool TB, int GROUP_M, int MIN_BLOCKS,
          int EDGE_MIN = 0, bool PF = false, int DIRECT = 0>
hipError_t launch_cfg(const Problem& p, int batch, hipStream_t stream, float* ws = nullptr, int slices = 1) {
  static_assert(BM == BN && BM % kEdge == 0, "square tiles whose sides are multiples of the edge tile");
  TileMap map;
  map.dp_tiles = map.sk_wgs = 0;
  map.ws = nullptr;
  map.slices = 1;
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
  long long edge_tiles = (long long)map.right_m * map.right_n + (long long)map.bottom_m * map.bottom_n;
  const dim3 block(WM * WN * KS * 64);
  const bool vec = vec_loads_ok(p, batch);
  if constexpr (BM == 64 && PF) {
    if (slices > 1 && ws != nullptr && batch == 1 && edge_tiles == 0 && nmfma > 0 &&
        nmfma * slices * (BM * BN) * 4 <= kStreamKBytes) {
      map.slices = slices;
      map.ws = ws;
      const long long blocks = nmfma * slices;
      if (!grid_fits(blocks, block.x)) return hipErrorInvalidConfiguration;
      if (vec)
        hipLaunchKernelGGL(
            (mfma_kernel<BM, BN, BK, WM, WN, KS, TA, TB, GROUP_M, MIN_BLOCKS, EDGE_MIN, false, true, PF, false, true>),
            dim3((unsigned)blocks), block, 0, stream, p, map);
      else
        hipLaunchKernelGGL(
            (mfma_kernel<BM, BN, BK, WM, WN, KS, TA, TB, GROUP_M, MIN_BLOCKS, EDGE_MIN, false, false, PF, false, true>),
            dim3((unsigned)blocks), block, 0, stream, p, map);
      const hipError_t err = hipGetLastError();
      if (err != hipSuccess) return err;
      hipLaunchKernelGGL((slice_fixup_kernel<BM, BN, GROUP_M>), dim3((unsigned)nmfma, BM), dim3(BN / 4 * kSliceGroups),
                         0, stream, p, map);
      return hipGetLastError();
    }
  }
  if constexpr (EDGE_MIN == 0 && BM == 256 && BN == 256) {  // the workspace holds 256 x 256 slots
    if (ws != nullptr && batch == 1 && nmfma % kStreamKWgs != 0) {
      // the partial wave, and the full wave before it where the partial one is under 1/8
      // of a wave (its pieces would be too short to fill the pipeline)
      const long long rem = nmfma % kStreamKWgs;
      const long long sk_tiles = rem + (nmfma > kStreamKWgs && rem < kStreamKWgs / 8 ? kStreamKWgs : 0);
      map.dp_tiles = (int)(nmfma - sk_tiles);
      map.sk_wgs = kStreamKWgs;
      map.ws = ws;
      const long long blocks = map.dp_tiles + map.sk_wgs + edge_tiles;
      if (!grid_fits(blocks, block.x)) return hipErrorInvalidConfiguration;
      if constexpr (DIRECT)
        hipLaunchKernelGGL(
            (mfma_kernel<BM, BN, BK, WM, WN, KS, TA, TB, GROUP_M, MIN_BLOCKS, 0, true, true, PF, false, false, DIRECT>),
            dim3((unsigned)blocks), block, 0, stream, p, map);
      else if (vec)
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
  // The right thin strip inside the tiles (FusedStrip, FUSE) in the 64 configuration, with
  // operands stored row-major, at least BM / 4 tile columns so that every strip row has its
  // tile, and K of at least kFuseMinK; otherwise the strip runs as thin-strip workgroups.
  // Fused, the strip adds a little to every K-tile of every tile and about 0.7 us to each
  // tile's end, against strip workgroups that take their own time per K (1000 x 1030 x 999:
  // 23.0 against 24.0 us; x 4000: 70.5 against 74.9 us; x 300: 11.6 against 10.9 us;
  // 1000 x 990 x 129: 8.6 against 7.8 us).  In the 128 configuration it measured slower
  // (2048 x 4100 x 2048: 253 against 249 us), in the 192 one no faster.  The direct K loop
  // with strip workgroups beats it (1000 x 1030 x 999: 22.0-22.1 against 22.8 us), so it
  // serves the register-staged loop only.
  constexpr int kFuseMinK = 640;
  constexpr int kThreadsPerWg = WM * WN * KS * 64;
  constexpr bool kCanFuse = BM == 64 && EDGE_MIN > 1 && PF && !TA && !TB && kThreadsPerWg == BK * 16 && !DIRECT;
  bool fuse = false;
  if constexpr (kCanFuse) {
    fuse = map.right_m > 0 && (long long)map.tiles_n * FusedStrip<BK, kThreadsPerWg>::SR >= BM && p.K >= kFuseMinK;
    if (fuse) {
      edge_tiles -= (long long)map.right_m * map.right_n;
      map.right_m = map.right_n = 0;
    }
  }
  const long long blocks = nmfma + edge_tiles;
  if (!grid_fits(blocks, block.x)) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)blocks, batch);
  if constexpr (kCanFuse) {
    if (fuse) {
      if (vec)
        hipLaunchKernelGGL(
            (mfma_kernel<BM, BN, BK, WM, WN, KS, TA, TB, GROUP_M, MIN_BLOCKS, EDGE_MIN, false, true, PF, true>), grid,
            block, 0, stream, p, map);
      else
        hipLaunchKernelGGL(
            (mfma_kernel<BM, BN, BK, WM, WN, KS, TA, TB, GROUP_M, MIN_BLOCKS, EDGE_MIN, false, false, PF, true>), grid,
            block, 0, stream, p, map);
      return hipGetLastError();
    }
  }
  if constexpr (DIRECT) {
    hipLaunchKernelGGL((mfma_kernel<BM, BN, BK, WM, WN, KS, TA, TB, GROUP_M, MIN_BLOCKS, EDGE_MIN, false, true, PF,
                                    false, false, DIRECT>),
                       grid, block, 0, stream, p, map);
  } else {
    if (vec)
      hipLaunchKernelGGL((mfma_kernel<BM, BN, BK, WM, WN, KS, TA, TB, GROUP_M, MIN_BLOCKS, EDGE_MIN, false, true, PF>),
                         grid, block, 0, stream, p, map);
    else
      hipLaunchKernelGGL((mfma_kernel<BM, BN, BK, WM, WN, KS, TA, TB, GROUP_M, MIN_BLOCKS, EDGE_MIN, false, false, PF>),
                         grid, block, 0, stream, p, map);
  }
  return hipGetLastError();
}

// The 16 configuration: one 16 x 16 block of C per workgroup of NT threads, over the whole
// K range split between its wavefronts, on 16 x 16 x 4 MFMA with operands loaded straight
// from global memory (thin_strip's block form, for whole blocks).  For products whose
// output is a few hundred such blocks: the larger tiles would run a handful of workgroups,
// each a latency-bound chain of K-tiles (256^3: 3.6 us against 4.5 us on 32 x 32 tiles;
// 256 x 256 x 1024: 5.8 against 8.7 us).  Block (bm, bn) is workgroup bm * blocks_n + bn.
constexpr int kBlock16Threads = 512;
template <int NT, bool TA, bool TB, bool VEC>
__global__ __launch_bounds__(NT) void block16_kernel(Problem p, int blocks_n) {
  p = batch_entry(p);
  __shared__ __attribute__((aligned(16))) float smem[thin_red_floats<NT>()];
  poison_lds(smem, thin_red_floats<NT>());
  const int bm = blockIdx.x / blocks_n, bn = blockIdx.x - (blockIdx.x / blocks_n) * blocks_n;
  const int first = bm * kThinMax, lo = bn * kThinMax;
  thin_strip<NT, TA, TB, VEC>(p, true, first, min(kThinMax, p.M - first), lo, min(kThinMax, p.N - lo), smem);
}

template <bool TA, bool TB>
hipError_t launch_block16(const Problem& p, int batch, hipStream_t stream) {
  constexpr int NT = kBlock16Threads;
  const long long bm = (p.M + kThinMax - 1) / kThinMax, bn = (p.N + kThinMax - 1) / kThinMax;
  if (!grid_fits(bm * bn, NT)) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)(bm * bn), batch), block(NT);
  if (vec_loads_ok(p, batch))
    hipLaunchKernelGGL((block16_kernel<NT, TA, TB, true>), grid, block, 0, stream, p, (int)bn);
  else
    hipLaunchKernelGGL((block16_kernel<NT, TA, TB, false>), grid, block, 0, stream, p, (int)bn);
  return hipGetLastError();
}

// The tile configurations (tile_plan.h), by tile side.  All but the 32 configuration run
// mfma_tile_pf (fragments read one K-tile ahead).
//   256: 256 x 256 tiles, BK 16, one workgroup per CU.  With the direct K loop (16-byte
//        aligned rows, direct_ok) 4 x 2 wavefronts of 64 x 128, two per SIMD (128
//        accumulator registers each); otherwise 2 x 2 wavefronts of 128 x 128, one per SIMD
//        (256 accumulator registers each), loads two K-tiles ahead through registers.
//   192: 192 x 192 tiles, 2 x 2 wavefronts of 96 x 96 (144 accumulator registers), BK 16,
//        one workgroup per CU: the direct K loop where direct_ok, else one global
//        register set.  Its tile counts fill whole waves where the others do not (3072^3:
//        256 tiles).
//   128: 128 x 128 tiles, 2 x 2 wavefronts of 64 x 64, BK 16, two workgroups per CU: the
//        direct K loop where direct_ok, else two global register sets.  At most one tile
//        per CU: 4 x 2 wavefronts of 32 x 64, one workgroup per CU, the same two loops.
//   64:  64 x 64 tiles, 2 x 2 wavefronts of 32 x 32 and a 2-way K split, BK 32, two
//        workgroups per CU: with more than one tile per CU the direct K loop where
//        direct_mask allows it, else two global register sets.
//   32:  32 x 32 tiles, one 32 x 32 block per wavefront and a 4-way K split, BK 64,
//        256 threads, mfma_tile; four workgroups per CU.
//   16:  16 x 16 blocks on 16 x 16 x 4 MFMA, K split over 8 wavefronts, no LDS staging
//        (block16_kernel).
// Partial tiles (mfma_edge_min): guarded MFMA tiles of the same grid in the 192, 128, 64
// and 32 configurations, except strips thinner than 16 in the 192, 128 and 64
// configurations (thin strips); in the 256 configuration the same on the direct K loop,
// else thin strips (both remainders under 16) or the scalar edge-tile path.
// ws: stream-K workspace (kStreamKBytes) for the 256 configuration, or for the 64 one's
// K slices (slices > 1), or nullptr.
template <bool TA, bool TB>
hipError_t launch_op(const Problem& p, int batch, hipStream_t stream, int tiles, float* ws = nullptr,
                     int slices = 1) {
  switch (tiles) {
    case 256:
      // Rows that LDS-DMA loads can read (direct_ok): the direct K loop on 4 x 2 wavefronts of 64 x 128, two per
      // SIMD (4096^3: 909 against 918 us on 2 x 2 wavefronts of 128 x 128, one per SIMD);
      // otherwise the register-staged loop on 2 x 2 wavefronts.
      // The direct loop also runs the partial tiles: remainders of at least kThin256 as guarded
      // tiles of the same grid, thinner ones as thin strips (4000^3: 892 against 947 us on
      // 128 x 128 tiles; 8000^3: 7089 against 7352 us on 192 x 192 tiles); full tiles only:
      // stream-K where a workspace is given.  The register-staged loop: remainders both
      // thinner than kThin256 as thin strips after the tiles (4100^3: see tile_plan.h),
      // wider ones as scalar edge tiles.
      if (direct_ok(p, batch)) {
        if (p.M % 256 != 0 || p.N % 256 != 0)
          return launch_cfg<256, 256, 16, 4, 2, 1, TA, TB, 8, 1, kThin256, true, true>(p, batch, stream);
        return launch_cfg<256, 256, 16, 4, 2, 1, TA, TB, 8, 1, 0, true, true>(p, batch, stream, ws);
      }
      if ((p.M % 256 != 0 || p.N % 256 != 0) && thin256(p.M, p.N))
        return launch_cfg<256, 256, 16, 2, 2, 1, TA, TB, 8, 1, kThin256, true>(p, batch, stream);
      return launch_cfg<256, 256, 16, 2, 2, 1, TA, TB, 8, 1, mfma_edge_min(256), true>(p, batch, stream, ws);
    case 192:
      // the direct K loop where the rows allow it: as fast as the register-staged loop with
      // operands along k (3072^3: 398.9 against 399.2 us), faster with A^T (398.1 against
      // 407.4 us)
      if (direct_ok(p, batch, 192)) {
        if (p.M % 192 == 0 && p.N % 192 == 0)
          return launch_cfg<192, 192, 16, 2, 2, 1, TA, TB, 8, 1, 0, true, true>(p, batch, stream);
        return launch_cfg<192, 192, 16, 2, 2, 1, TA, TB, 8, 1, mfma_edge_min(192), true, true>(p, batch, stream);
      }
      if (p.M % 192 == 0 && p.N % 192 == 0)
        return launch_cfg<192, 192, 16, 2, 2, 1, TA, TB, 8, 1, 0, true>(p, batch, stream);
      return launch_cfg<192, 192, 16, 2, 2, 1, TA, TB, 8, 1, mfma_edge_min(192), true>(p, batch, stream);
    case 128: {
      // At most one tile per CU: the second workgroup slot of a CU would stay empty, so
      // the tile takes 4 x 2 wavefronts of 32 x 64, two per SIMD, each covering the
      // other's barrier waits (2048^3: 123.0 us, against 125.2 with 2 x 2 wavefronts and
      // BK 32, and 127.7 with the two-workgroup form; guarded tiles, 1900^3: 116.1 against
      // 121.0 us).  With more tiles the two-workgroup form is as fast or faster (4000^3:
      // 941 against 956 us for BK 32 at one workgroup per CU).  Both forms run the direct K
      // loop where the rows allow it (two-workgroup form, 4096^3: 931 against 966 us;
      // 2048 x 4096 x 4096: 474 against 488; one-layer form, 2048^3: 122.4 against 123.7
      // us), with the operands stored along m or n in the packed layout (one load per two
      // k-rows): with one k-row per load on half the lanes, the one-layer form ran slower
      // than through registers (124.2 against 123.9 us), and so did A^T (2048 x 4096 x
      // 4096 TN: 500 against 487 us; packed: 469 against 488).
      constexpr int em = mfma_edge_min(128);
      const bool exact = p.M % 128 == 0 && p.N % 128 == 0;
      const long long tiles = (long long)((mfma_extent(p.M, 128, exact ? 0 : em) + 127) / 128) *
                              ((mfma_extent(p.N, 128, exact ? 0 : em) + 127) / 128) * batch;
      if (tiles <= kCUs && (direct_mask(p, batch) & kDirect128))
        return exact ? launch_cfg<128, 128, 16, 4, 2, 1, TA, TB, 8, 1, 0, true, true>(p, batch, stream)
                     : launch_cfg<128, 128, 16, 4, 2, 1, TA, TB, 8, 1, em, true, true>(p, batch, stream);
      if (tiles <= kCUs)
        return exact ? launch_cfg<128, 128, 16, 4, 2, 1, TA, TB, 8, 1, 0, true>(p, batch, stream)
                     : launch_cfg<128, 128, 16, 4, 2, 1, TA, TB, 8, 1, em, true>(p, batch, stream);
      if (direct_mask(p, batch) & kDirect128)
        return exact ? launch_cfg<128, 128, 16, 2, 2, 1, TA, TB, 8, 2, 0, true, true>(p, batch, stream)
                     : launch_cfg<128, 128, 16, 2, 2, 1, TA, TB, 8, 2, em, true, true>(p, batch, stream);
      return exact ? launch_cfg<128, 128, 16, 2, 2, 1, TA, TB, 8, 2, 0, true>(p, batch, stream)
                   : launch_cfg<128, 128, 16, 2, 2, 1, TA, TB, 8, 2, em, true>(p, batch, stream);
    }
    case 64: {
      // The direct K loop where the rows allow it (K a multiple of 32): 2560^3 267 against
      // 285 us, 4608^3 1455 against 1518 (before the packed layout), 2560^3 TN 272 against
      // 313; at one tile per CU 1024^3 19.3-19.7 against 20.0-20.1 us (with one k-row of B
      // per load it had been slower there: 20.3 against 19.9).
      constexpr int em = mfma_edge_min(64);
      const bool exact = p.M % 64 == 0 && p.N % 64 == 0;
      if (direct_mask(p, batch) & kDirect64) {
        if (p.K % 32 != 0)  // the partial last K-tile through registers
          return exact ? launch_cfg<64, 64, 32, 2, 2, 2, TA, TB, 8, 2, 0, true, 2>(p, batch, stream, ws, slices)
                       : launch_cfg<64, 64, 32, 2, 2, 2, TA, TB, 8, 2, em, true, 2>(p, batch, stream, ws, slices);
        return exact ? launch_cfg<64, 64, 32, 2, 2, 2, TA, TB, 8, 2, 0, true, true>(p, batch, stream, ws, slices)
                     : launch_cfg<64, 64, 32, 2, 2, 2, TA, TB, 8, 2, em, true, true>(p, batch, stream, ws, slices);
      }
      return exact ? launch_cfg<64, 64, 32, 2, 2, 2, TA, TB, 8, 2, 0, true>(p, batch, stream, ws, slices)
                   : launch_cfg<64, 64, 32, 2, 2, 2, TA, TB, 8, 2, em, true>(p, batch, stream, ws, slices);
    }
    case 32:
      if (p.M % 32 == 0 && p.N % 32 == 0) return launch_cfg<32, 32, 64, 1, 1, 4, TA, TB, 8, 4>(p, batch, stream);
      return launch_cfg<32, 32, 64, 1, 1, 4, TA, TB, 8, 4, mfma_edge_min(32)>(p, batch, stream);
    case 16:
      return launch_block16<TA, TB>(p, batch, stream);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace mfma_detail
}  // namespace sgemm_impl
