// Choice of the MFMA tile configuration for a problem (host code).
//
// A launch of T tiles (over the whole batch) gives each of the 256 CUs up to
// ceil(T / 256) tiles, each costing time proportional to K.  The time of a
// configuration is modelled as ceil(T / 256) * K * u, with u its measured time per
// tile and unit of K on a CU that holds one tile (u1) or several (u2); the model
// picks the configuration with the least time.  The per-configuration figures come
// from a sweep of square and rectangular shapes on MI355X (microseconds per 1024 of
// K per tile-layer, net of about 5 us of launch cost); they reproduce the measured
// times of every configuration within about 10% on shapes whose tiles are full or
// guarded.  Thin strips (remainders under 16 in the 128 and 64 configurations) run
// beside the tiles and are not counted; they add up to about 10% at long K (4100^3 on
// 128 x 128 tiles: 992 us against 957 us at 4096^3).  Transposed operands use the same
// figures.
#pragma once

#include "internal.h"

namespace sgemm_impl {

struct TileCost {
  int side;  // tile side: 256, 192, 128, 64, 32 or 16
  double u1, u2;
  double thin;  // us per 1024 of K per 256 thin-strip workgroups
};
// Thin strips are priced in the 32 configuration, whose tiles fill all four workgroup slots
// of a CU, and in the 256 one, whose workgroups each take a whole CU: there the strips run
// after the tiles (a strip workgroup takes about 3.3 us per 1024 of K on its own); beside
// the other configurations' tiles they overlap.  Fitted together with the
// tile costs against forced-configuration timings of 75 shapes (squares, skinny, long-K,
// ragged, batched, and 40 seeded random ones): the choice costs 0.5% on average against
// the fastest configuration of each shape.
// The 16 configuration's blocks (one per workgroup of 8 wavefronts) read their operands
// straight from global memory, without the tiles' reuse through LDS, so their cost grows
// with the blocks in flight as well as with the layers: kBlock16Base + kBlock16PerBlock B
// us per 1024 of K for one layer of B <= 256 blocks, kBlock16Layer per layer beyond (a fit
// to eager timings of 120 seeded random shapes, every configuration forced: 2.6 us for any
// layer before, which chose 16 x 16 blocks over 32 x 32 tiles where those were up to 1.5x
// faster, e.g. 3057 x 61 x 573, 768 blocks: 11.1 against 7.5 us; mean loss against the
// fastest configuration 2.0% -> 1.6%).  The kTileCosts entry of side 16 is not used.
constexpr double kBlock16Base = 2.5, kBlock16PerBlock = 0.006, kBlock16Layer = 4.0;
constexpr TileCost kTileCosts[] = {{256, 231.0, 231.0, 4.0},
                                   {192, 134.0, 133.3, 0.0},
                                   {128, 60.5, 59.5, 0.0},
                                   {64, 15.3, 16.0, 0.0},
                                   {32, 5.4, 4.95, 4.0},
                                   {16, 2.6, 2.8, 0.0}};
// The direct K loops (direct_ok), priced relative to the register-staged ones they
// replace.  128 configuration, two-workgroup form: u2 3.3% below the staged loop's (net of
// launch cost, the mean of six shapes timed both ways on one box: 4096^3 931 against 966
// us, 2048 x 4096 x 4096 474 / 488, 4096 x 2048 x 2048 237 / 247, 2816^3 326 / 337,
// 1024 x 8192 x 1024 122.9 / 126.7, 7168^3 5386 / 5521).  256 configuration (4 x 2
// wavefronts): 4096^3 906-908 us against 963-966 on staged 128 x 128 tiles on the same
// boxes, i.e. 0.941 of the 128 configuration's modelled time there.
// 64 configuration, two-workgroup form: u2 4.4% below the staged loop's on one box (2560^3
// 273.5 against 284.6 us, 3584^3 701 / 732, 4608^3 1455 / 1518, 2304^3 211.8 / 221.7,
// 1536 x 4096 x 4096 374 / 388: 15.3), 15.7-16.4 on another (eight squares and
// rectangles from 2560 to 7168, next to 57.4-60.3 for the 128 form there), with B loaded
// one k-row per instruction; with B in the packed layout 3% less again (2560^3 267 against
// 276 us).
// At one tile per CU the 64 configuration's direct loop (packed layout) runs 1024^3 in
// 19.3-19.7 against 20.0-20.1 us: u1 3% below.
constexpr double kDirect128U2 = 57.5, kDirect256U = 224.0, kDirect64U2 = 15.2, kDirect64U1 = 14.85;

// MFMA tiles along one dimension of n.  A partial strip that runs as guarded MFMA tiles
// counts as a tile row (column); a thin strip, which runs beside the MFMA tiles, does not.
inline long long modelled_tiles(int n, int side, int edge_min) {
  return (mfma_extent(n, side, edge_min) + side - 1) / side;
}

// Thin-strip workgroups (16 lines each) of one product, for B stored along n (the last
// 1-3 columns of a guarded remainder that is not a multiple of 4 are thin too).
inline long long modelled_thin_wgs(int M, int N, int side) {
  const int em = side == 256 ? kThin256 : mfma_edge_min(side);
  if (em <= 1) return 0;
  const int Mf = mfma_extent(M, side, em), Nf = mfma_extent(N, side, em) & ~3;
  return (Nf < N ? (Mf + 15) / 16 : 0) + (Mf < M ? (N + 15) / 16 : 0);
}

// Modelled microseconds; M, N, K, batch > 0.  direct: the configurations whose direct K
// loops run the problem (direct_mask): the 256 configuration and the 128 and 64 ones'
// two-workgroup forms then cost kDirect256U, kDirect128U2 and kDirect64U2, and the 256
// configuration runs guarded tiles too (4000^3:
// 892 us against 947 on 128 x 128 tiles; 3900 x 3900 x 3904: 871 against 933; 8000^3:
// 7089 against 7352 on 192 x 192 tiles, while the model keeps 192 for 3000 x 3000 x 3008,
// 394 us against 670 on guarded 256 tiles, whose one layer of 144 tiles leaves CUs idle).
// Without it the 256 configuration is a candidate only where its tiles cover the matrix,
// or leave remainders thinner than kThin256 over one layer of tiles (thin strips after
// the tiles: 4096 x 4100 x 4096 940 us against 969 on 128 x 128 tiles; 4100^3 980 against
// 993, which the model still gives to 128).  Wider strips would run as scalar edge tiles, which
// cannot share a CU with its workgroups and are latency-bound chains of K-steps (4000^3:
// 1434 us, against 949 us on 128 x 128 tiles; 4090^3: 1887 against 1021 us).  A guarded
// 256 x 256 tile costs a whole tile, as in the other configurations.
inline double modelled_time(const TileCost& c, int M, int N, int K, int batch, int direct = 0) {
  const bool d256 = (direct & kDirect256) != 0;
  if (c.side == 256 && !d256 && !thin256(M, N)) return 1e30;
  const int em = c.side == 256 ? (d256 ? kThin256 : 0) : mfma_edge_min(c.side);
  const long long tiles = modelled_tiles(M, c.side, em) * modelled_tiles(N, c.side, em) * batch;
  const long long layers = (tiles + 255) / 256;
  if (c.side == 16)
    return (layers == 1 ? kBlock16Base + kBlock16PerBlock * (double)tiles : kBlock16Layer * (double)layers) *
           (double)K / 1024.0;
  // thin strips in the 256 configuration only over one layer of tiles: past it the strips'
  // workgroups, each on a whole CU, add up (8200^3: 7809 against 7773 us on 128 x 128 tiles)
  const long long thin_wgs = modelled_thin_wgs(M, N, c.side);
  if (c.side == 256 && thin_wgs > 0 && layers > 1) return 1e30;
  const long long thin_rounds = (thin_wgs * batch + 255) / 256;
  const double u1 = c.side == 256 && d256                      ? kDirect256U
                    : c.side == 64 && (direct & kDirect64) != 0 ? kDirect64U1
                                                                 : c.u1;
  const double u2 = c.side == 256 && d256                       ? kDirect256U
                    : c.side == 128 && (direct & kDirect128) != 0 ? kDirect128U2
                    : c.side == 64 && (direct & kDirect64) != 0   ? kDirect64U2
                                                                  : c.u2;
  return ((double)layers * (layers > 1 ? u2 : u1) + (double)thin_rounds * c.thin) * (double)K / 1024.0;
}

// Stream-K (256 configuration, batch 1, with a workspace, full tiles only): the K-tiles of
// the last partial wave of T full tiles (and of the full wave before it where the partial
// one holds fewer than 32 tiles) are shared evenly by 256 workgroups, so the MFMA time is
// T/256 layers instead of ceil(T/256), at
// kStreamKCost (the stream-K instantiation runs the tile code as an outlined function,
// about 2% slower per K-tile than the one-tile kernel), plus a fixed cost of about 110 us:
// each workgroup's two partial pieces (pipeline fill and 256 KB partial-tile stores) and
// the fix-up pass (about 45 us for 300 split tiles).  Measured (us, stream-K against the
// model): 4352 x 4096 x 4096 1079 / 1113, x 8192 2067 / 2116, 4608^3 1423 / 1454, 5120^3
// 1911 / 1954, 6144^3 3227 / 3296.  On the direct K loop (direct: direct_ok; its tile
// code inlined into the stream-K kernel) the pieces cost less: 4352 x 4096 x 4096 1020 us,
// 4608^3 1333, 5120^3 1822 (a least-squares fit gives 226 us per layer-1024 and 56 us).
// With fewer than 256 tiles every tile is split and the pieces' overheads dominate, so
// stream-K is a candidate only past one full wave.  Returns a negative value where it does
// not apply.
constexpr double kStreamKCost = 236.0, kStreamKOverhead = 110.0;               // us per layer-1024, us
constexpr double kDirectStreamKCost = 228.0, kDirectStreamKOverhead = 50.0;  // on the direct K loop
inline double modelled_stream_k_time(int M, int N, int K, int batch, bool direct = false) {
  const long long tiles = (long long)(M / 256) * (N / 256);
  if (batch != 1 || M % 256 != 0 || N % 256 != 0) return -1.0;
  if (tiles <= kStreamKWgs || tiles % kStreamKWgs == 0) return -1.0;
  return (double)tiles / kStreamKWgs * (direct ? kDirectStreamKCost : kStreamKCost) * (double)K / 1024.0 +
         (direct ? kDirectStreamKOverhead : kStreamKOverhead);
}

// K slices (64 configuration, batch 1, with a workspace): a product of few tiles and long K
// leaves most CUs idle however its tiles are cut; its K range can be cut instead.  Each of
// the tiles' K ranges is split into S contiguous slices, one workgroup each, so that the
// launch holds about one workgroup per CU with at least kMinSliceIters K-tiles of 32 per
// slice (about two per CU measured 2-24% slower on 6 of 8 shapes, e.g. 64 x 64 x 262144:
// 38.3 against 30.7 us, 512 x 512 x 16384: 80.7 against 74.3 us; faster on 1024 x 64 x
// 65536: 85.6 against 90.8 us); the raw partial tiles go to the workspace
// and a second kernel adds them in slice order (deterministic) and applies alpha and beta.
// Thin strips do not split, so the form applies where the 64 configuration's tiles cover
// the matrix (remainders of 0 or at least 16 rows, and of 0 or at least 16 columns that
// are a multiple of 4).  Returns S, or 1 where slicing does not apply.
constexpr int kMinSliceIters = 16;
inline int k_slices(int M, int N, int K, int batch) {
  if (batch != 1 || M <= 0 || N <= 0 || K <= 0) return 1;
  const bool covered = (M % 64 == 0 || M % 64 >= 16) && (N % 64 == 0 || (N % 64 >= 16 && N % 4 == 0));
  if (!covered) return 1;
  const long long tiles = (long long)((M + 63) / 64) * ((N + 63) / 64);
  const long long iters = (K + 31) / 32;
  long long s = kCUs / tiles;
  if (s > iters / kMinSliceIters) s = iters / kMinSliceIters;
  return s >= 2 ? (int)s : 1;
}
// Modelled time of the sliced form: the layer of tiles x S workgroups at the 64
// configuration's cost over K / S, plus the fix-up (a launch and the partial tiles read
// at about 2 TB/s); negative where it does not apply.
constexpr double kSliceFixupUs = 3.0;
inline double modelled_sliced_time(int M, int N, int K, int batch) {
  const int S = k_slices(M, N, K, batch);
  if (S < 2) return -1.0;
  const long long tiles = (long long)((M + 63) / 64) * ((N + 63) / 64);
  const long long layers = (tiles * S + kCUs - 1) / kCUs;
  static_assert(kTileCosts[3].side == 64, "the 64 configuration's costs");
  const TileCost& c64 = kTileCosts[3];
  const double part_bytes = (double)tiles * S * 64 * 64 * 4;
  return (double)layers * (layers > 1 ? c64.u2 : c64.u1) * ((double)K / S) / 1024.0 + kSliceFixupUs +
         part_bytes / 2.0e6;
}

struct TilePlan {
  int side;        // tile configuration
  bool stream_k;   // stream-K over the last waves (side 256 only)
  int slices = 1;  // K slices (side 64 only; k_slices)
};

// The configuration with the least modelled time (ties: the larger tile); stream-K and K
// slices are candidates when a workspace is available; direct as modelled_time's.
inline TilePlan plan_tiles(int M, int N, int K, int batch, bool workspace = false, int direct = 0) {
  TilePlan best{kTileCosts[0].side, false};
  double t = modelled_time(kTileCosts[0], M, N, K, batch, direct);
  for (const TileCost& c : kTileCosts) {
    const double tc = modelled_time(c, M, N, K, batch, direct);
    if (tc < t) best = TilePlan{c.side, false}, t = tc;
  }
  if (workspace) {
    const double tsk = modelled_stream_k_time(M, N, K, batch, (direct & kDirect256) != 0);
    if (tsk >= 0.0 && tsk < t) best = TilePlan{256, true}, t = tsk;
    const double tsl = modelled_sliced_time(M, N, K, batch);
    if (tsl >= 0.0 && tsl < t) best = TilePlan{64, false, k_slices(M, N, K, batch)}, t = tsl;
  }
  return best;
}

}  // namespace sgemm_impl
