// Choice of the MFMA tile configuration for a problem (host code).
//
// A launch of T tiles (over the whole batch) gives each of the 256 CUs up to
// ceil(T / 256) tiles, each costing time proportional to K.  The time of a
// configuration is modelled as ceil(T / 256) * K * u, with u its measured time per
// tile and unit of K on a CU that holds one tile (u1) or several (u2); the model
// picks the configuration with the least time.  The per-configuration figures come
// from a sweep of square and rectangular shapes on MI355X (microseconds per 1024 of
// K per tile-layer, net of about 5 us of launch cost); they reproduce the measured
// times of every configuration within about 10%.  Transposed operands use the
// same figures.
#pragma once

#include "internal.h"

namespace sgemm_impl {

struct TileCost {
  int side;  // tile side: 256, 128, 64 or 32
  double u1, u2;
};
constexpr TileCost kTileCosts[] = {{256, 237.0, 237.0}, {128, 64.7, 64.7}, {64, 16.2, 17.2}, {32, 5.4, 4.95}};

// M, N, K, batch > 0.
inline double modelled_time(const TileCost& c, int M, int N, int K, int batch) {
  const long long tiles = ((long long)(M - 1) / c.side + 1) * ((long long)(N - 1) / c.side + 1) * batch;
  const long long layers = (tiles + 255) / 256;
  return (double)layers * (layers > 1 ? c.u2 : c.u1) * (double)K;
}

// Tile side of the configuration with the least modelled time (ties: the larger tile).
inline int plan_tiles(int M, int N, int K, int batch) {
  int best = kTileCosts[0].side;
  double t = modelled_time(kTileCosts[0], M, N, K, batch);
  for (const TileCost& c : kTileCosts) {
    const double tc = modelled_time(c, M, N, K, batch);
    if (tc < t) best = c.side, t = tc;
  }
  return best;
}

}  // namespace sgemm_impl
