// MFMA SGEMM, the direct-to-LDS K loop (the 256, 192, 128 and 64 configurations): the
// operands of each K-tile go from global memory straight into an LDS stage
// (buffer_load_dwordx4 ... lds, gfx950's 128-bit LDS-DMA load), with no register staging
// and no LDS store instructions.
#pragma once

#include <type_traits>
#include "mfma_tiles.h"

namespace sgemm_impl {
namespace mfma_detail {

// LDS stages of the direct pipeline (4 x 32.25 KiB in the 256 configuration, 4 x 16.5 KiB
// in the 64 one, whose 5 or 6 stages measured slower: 1024^3 19.4 and 19.6 against 19.1
// us).  A K-tile is loaded NST K-tiles ahead
// of its MFMAs, and the wait before each barrier leaves the last NST - 2 K-tiles' loads in
// flight.  Measured at 4096^3 (a standalone copy on 2 x 2 wavefronts, one load per 1 or 2
// MFMAs): 3 stages 922, 4 stages 913-915 us.
constexpr int kDirectStages = 4;
// One load instruction after every kDirectSpacing-th MFMA of a K-tile.  4096^3 on 2 x 2
// wavefronts (8 loads, 128 MFMAs per wavefront and K-tile), two runs: after every 1st, 2nd,
// 4th MFMA 914.6, 913.4, 913.2 us; every 4th, 8th, 16th 909.4, 914.5, 918.5 us; all eight
// loads before the MFMAs 950.3 us.  On 4 x 2 wavefronts (4 loads, 64 MFMAs): every 4th or
// 8th 909.1 and 908.5 us.  The smaller tiles take one after every 2nd (1024^3 on 64 x 64
// tiles: 19.0-19.1 against 19.3 us; 2048^3 on 128 x 128: 121.1 against 121.6; 2560^3 on
// 64 x 64: 265.6 against 264.8).
constexpr int kDirectSpacing = 4, kDirectSpacingSmall = 2;

typedef int v4i __attribute__((ext_vector_type(4)));

// x, the same in every lane, as a value the compiler knows to be uniform (scalar
// registers): address arithmetic on it then stays on the scalar unit.
__device__ __forceinline__ long long uniform64(long long x) {
  const unsigned lo = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)x);
  const unsigned hi = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)((unsigned long long)x >> 32));
  return (long long)(((unsigned long long)hi << 32) | lo);
}

// Buffer resource of a raw buffer at `base` (64-bit address, stride 0, no range limit
// below 2^31 bytes; gfx9 data format word).  `base` is uniform; computed from uniform64
// values it is already in scalar registers and the readfirstlanes fold away.
__device__ __forceinline__ v4i buffer_rsrc(const float* base) {
  const long long a = uniform64(reinterpret_cast<long long>(base));
  return v4i{(int)(unsigned)a, (int)(unsigned)((unsigned long long)a >> 32), 0x7fffffff, 0x00020000};
}

// Byte address of p inside the workgroup's LDS.
__device__ __forceinline__ unsigned lds_address(const float* p) {
  return (unsigned)reinterpret_cast<unsigned long long>((__attribute__((address_space(3))) const float*)p);
}

// One 128-bit LDS-DMA load: lane l reads 16 bytes at base + voff and writes them to LDS
// bytes [lds + 16 l, lds + 16 l + 16).  Written as inline assembly: the compiler treats
// its own LDS-DMA loads as LDS writes of unknown address and waits for all of them before
// every LDS read, which would serialise the pipeline; here the waits are explicit
// (direct_barrier).  s_nop 4: five wait states between a VALU write of an SGPR operand
// and the load's read of it; s_nop 0 after the M0 write, before the load reads M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_dma16(v4i rsrc, unsigned lds, unsigned voff) {
  asm volatile(
      "s_nop 4\n\t"
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(__builtin_amdgcn_readfirstlane((int)lds)),
      "v"(voff), "s"(rsrc)
      : "memory", "m0");
}
#pragma clang diagnostic pop

// Wait until at most N vector-memory instructions of this wavefront are outstanding and
// all its LDS operations are done, then the workgroup barrier.
template <int N>
__device__ __forceinline__ void direct_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
  __builtin_amdgcn_sched_barrier(0);
}

template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (N > 0) {
    static_for<N - 1>(f);
    f(std::integral_constant<int, N - 1>{});
  }
}

// One R x BK operand slice (R a multiple of 64 up to 256, BK 16 or 32) loaded by LDS-DMA
// by W wavefronts: its stage layout is Operand's, so the fragment reads are unchanged.  NI
// loads per K-tile; wavefront w issues L = NI / W of them, load i being load j = L w + i:
//   KROWS (A, or B^T): NI = R BK / 256; load j fills the RPI = 256 / BK rows from RPI j
//     (1 KiB), KC = BK / 4 16-byte chunks each; lane l takes row RPI j + l / KC at chunk
//     position l % KC, which holds the chunk that swz_slot puts there (position XOR the
//     row's swizzle: for BK 16, (l % 4) ^ (l / 16));
//   otherwise (A^T, or B): NI = BK; load j fills k-row j, R floats, lane l < R/4 taking
//     floats 4l .. 4l+3 (the other lanes are masked off; the row's 4 padding words stay
//     unwritten and unread: the form of R = 256, where every lane loads; with fewer lanes
//     it ran slower than register staging); PACKED (Operand's packed layout, R < 256):
//     NI = R BK / 256, load j filling floats 256 j .. 256 j + 255 of the stage (256 / R
//     k-rows, or parts of two), every lane loading the 4 floats that kslot puts at its 16
//     bytes.
// GUARD (a tile reaching past M or N): lines at or past lim, the slice's lines inside the
// matrix, load the last row (KROWS) or the last float4 inside (otherwise; lim is then a
// multiple of 4), as Operand::load_full does: their values reach only outputs that are not
// stored.
template <int R, int BK, bool KROWS, int W, bool PACKED = false>
struct DirectOperand {
  static constexpr int KC = BK / 4, RPI = 256 / BK, NI = KROWS || PACKED ? R * BK / 256 : BK, L = NI / W;
  static constexpr int kLanes = KROWS || PACKED ? 64 : R / 4;  // lanes that load
  static_assert(R % 64 == 0 && R <= 256 && (BK == 16 || BK == 32) && L * W == NI,
                "the loads split evenly over the wavefronts");
  using Op = Operand<R, BK, 64 * W, KROWS, PACKED>;
  const float* base;  // element (r0, k = 0) of the tile's slice
  long long kstep;    // floats between consecutive K-tiles
  unsigned voff[L];   // byte offsets of this lane's 16 bytes from the K-tile's origin
  unsigned lds[L];    // stage-relative LDS byte offsets of the wavefront's loads
  bool active;        // this lane loads (l < kLanes)

  template <bool GUARD>
  __device__ __forceinline__ void init(const float* X, long long ld, int r0, int rows_left, int w, int l) {
    // uniform: the K-tile origins base + kt * kstep are then computed by scalar instructions
    // (as vector ones, followed by readfirstlane, the loop ran 2% slower)
    base = reinterpret_cast<const float*>(
        uniform64(reinterpret_cast<long long>(KROWS ? X + (long long)r0 * ld : X + r0)));
    kstep = uniform64(KROWS ? BK : BK * ld);
    const int lim = rows_left < R ? rows_left : R;
    active = l < kLanes;
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const int j = L * w + i;
      if (KROWS) {
        const int row = RPI * j + l / KC, pos = l % KC;
        const int chunk = pos ^ ((swz_slot<BK>(row, 0) - row * BK) / 4);  // the row's XOR
        const int r = (!GUARD || row < lim) ? row : lim - 1;
        voff[i] = (unsigned)((long long)r * ld + 4 * chunk) * 4u;
        lds[i] = (unsigned)(RPI * j * BK) * 4u;
      } else if (PACKED) {
        // float 256 j + 4 l of the stage: k-row k, column position p, whose 16 bytes hold the
        // lines that kslot stores there
        const int k = (256 * j + 4 * l) / R, p = (256 * j + 4 * l) % R;
        const int c = min(p ^ (((k >> 3) & 1) << 5), (GUARD ? lim : R) - 4);
        voff[i] = (unsigned)((long long)k * ld + c) * 4u;
        lds[i] = (unsigned)(256 * j) * 4u;
      } else {
        const int c = min(4 * l, (GUARD ? lim : R) - 4);
        voff[i] = (unsigned)((long long)j * ld + c) * 4u;
        lds[i] = (unsigned)(j * Op::STRIDE) * 4u;
      }
    }
  }
  // load i of K-tile kt into the stage at LDS byte address `stage`
  __device__ __forceinline__ void load(int i, int kt, unsigned stage) const {
    const v4i rsrc = buffer_rsrc(base + (long long)__builtin_amdgcn_readfirstlane(kt) * kstep);
    if (kLanes == 64 || active) lds_dma16(rsrc, stage + lds[i], voff[i]);
  }
};

// K-tiles [kb, ke) of the BM x BM tile at (m0, n0), as mfma_tile_pf with WM x WN x KS
// wavefronts (256: 4 x 2, two per SIMD, each 64 x 128; 192: 2 x 2 of 96 x 96; 128: 4 x 2
// of 32 x 64, or 2 x 2 of 64 x 64 at two workgroups per CU; 64: 2 x 2 of 32 x 32 with a
// 2-way K split, two workgroups per CU), with kDirectStages LDS stages filled by LDS-DMA
// loads.  Tile j lives in stage (j - kb) % NST and fragment set
// (j - kb) % 2.  During K-tile t:
//   - tile t + NST is loaded into stage t's (its fragments were read during K-tile t - 1,
//     before the last barrier), one load after every SP-th MFMA;
//   - the fragments of tile t + 1 are read from its stage into the other set;
//   - the MFMAs of tile t run on their set;
// and before the barrier that ends it, each wavefront waits for its loads of tile t + 2
// (the last NST - 2 K-tiles' loads stay in flight), so that after the barrier tile t + 2
// is in LDS for every wavefront.  Every K-tile is whole (direct_ok) but, with TAIL, the
// last (below).  GUARD: as mfma_tile_pf's (bit 0 A rows past M, bit 1 B columns past N,
// bit 2 a launch of full tiles only).
template <int BM, int BK, int WM, int WN, int KS, bool TA, bool TB, int GUARD, bool TAIL = false>
__device__ __forceinline__ void mfma_tile_direct(const Problem& p, int m0, int n0, int kb, int ke, float* smem,
                                                 float* part) {
  constexpr int BN = BM, NST = kDirectStages, W = WM * WN * KS;
  // operands stored along m or n in Operand's packed layout below 256 (one load per 256 / BM
  // k-rows, every lane loading, instead of one per k-row on BM / 4 lanes)
  constexpr bool kPacked = BM < 256;
  using Cfg = MfmaCfg<BM, BN, BK, WM, WN, KS, TA, TB, kPacked>;
  using OpA = typename Cfg::OpA;
  using OpB = typename Cfg::OpB;
  using DA = DirectOperand<BM, BK, !TA, W, kPacked && TA>;
  using DB = DirectOperand<BN, BK, TB, W, kPacked && !TB>;
  constexpr int FM = Cfg::FM, FN = Cfg::FN, KG = Cfg::KG;
  static_assert(NST * Cfg::kStageFloats * 4 <= 160 * 1024, "stages fit the LDS");
  constexpr int kLoads = DA::L + DB::L;  // LDS-DMA loads per wavefront and K-tile
  constexpr int kMfmas = 8 * KG * FM * FN;
  // one load after every SP-th MFMA, all of them during the K-tile's MFMAs
  constexpr int kSpacing = BM == 256 ? kDirectSpacing : kDirectSpacingSmall;
  constexpr int SP = kLoads <= 1                                 ? kSpacing
                     : (kMfmas - 1) / (kLoads - 1) < kSpacing ? (kMfmas - 1) / (kLoads - 1)
                                                                : kSpacing;
  static_assert(SP >= 1 && (kLoads - 1) * SP < kMfmas, "the loads go out during the K-tile's MFMAs");
  auto a_stage = [&](int s) { return smem + s * Cfg::kStageFloats; };
  auto b_stage = [&](int s) { return smem + s * Cfg::kStageFloats + OpA::kStageFloats; };

  const int t = threadIdx.x, l = t % 64;
  const int w = __builtin_amdgcn_readfirstlane(t / 64);
  const int lr = l % 32, lh = l / 32;
  // K-group and spatial position of this wavefront
  const int ks = KS == 1 ? 0 : w / (WM * WN), sp = KS == 1 ? w : w % (WM * WN);
  const int wm0 = (sp / WN) * (BM / WM), wn0 = (sp % WN) * (BN / WN);

  DA da;
  DB db;
  da.template init<(GUARD & 1) != 0>(p.A, p.lda, m0, p.M - m0, w, l);
  db.template init<(GUARD & 2) != 0>(p.B, p.ldb, n0, p.N - n0, w, l);
  const unsigned lds0 = lds_address(smem);
  auto load_one = [&](int q, int kt, int s) {  // load q (A's, then B's) of full K-tile kt
    const unsigned stage = lds0 + (unsigned)(s * Cfg::kStageFloats) * 4u;
    if (q < DA::L)
      da.load(q, kt, stage);
    else
      db.load(q - DA::L, kt, stage + OpA::kStageFloats * 4u);
  };
  // K-tile kt into stage s
  auto fill = [&](int kt, int s) {
#pragma unroll
    for (int q = 0; q < kLoads; ++q) load_one(q, kt, s);
  };

  v16f acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  float af[2][KG][FM][8], bf[2][KG][FN][8];
  auto frags = [&](auto set, int s) {
    constexpr int S = decltype(set)::value;
#pragma unroll
    for (int r = 0; r < KG; ++r) {
      read_frags<OpA, FM, Cfg::VA>(a_stage(s), wm0, ks * KG + r, lr, lh, af[S][r]);
      read_frags<OpB, FN, Cfg::VB>(b_stage(s), wn0, ks * KG + r, lr, lh, bf[S][r]);
    }
  };
  auto mfma = [&](auto set, auto mc) {
    constexpr int S = decltype(set)::value, m = decltype(mc)::value;
    constexpr int r = m / (8 * FM * FN), e = (m / (FM * FN)) % 8, i = (m / FN) % FM, j = m % FN;
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[S][r][i][e], bf[S][r][j][e], acc[i][j], 0, 0, 0);
  };
  using Set0 = std::integral_constant<int, 0>;
  using Set1 = std::integral_constant<int, 1>;

  // TAIL (a launch whose K is not a multiple of BK, one whole tile per workgroup): the
  // partial last K-tile goes through registers, loaded after the prologue's fill (issued
  // at the start they delayed it: 1000 x 1030 x 999 22.1 against 21.9 us) with zeros past
  // K (Operand::load_tail; the loads are unconditional, since loads under a branch would be
  // waited for where it joins: a range that ended before it would load the last full
  // K-tile, unused) and stored to stage 0 after the direct loop.
  constexpr bool kTail = TAIL;
  const int nfull = p.K / BK;
  const bool tail = kTail && ke > nfull;
  const int kend = tail ? nfull : ke;  // the direct loop's K-tiles: [kb, kend)
  OpA tail_a;
  OpB tail_b;
  if constexpr (kTail) {
    tail_a.init(p.A, p.lda, m0, p.M - m0, t);
    tail_b.init(p.B, p.ldb, n0, p.N - n0, t);
  }

  // prologue: tiles kb .. kb + NST - 1 into stages 0 .. NST - 1; tile kb's fragments
  const int n = kend - kb;
  if (!kTail || n > 0) {  // n == 0: a partial K-tile alone
    for (int j = 0; j < NST; ++j)
      if (j < n) fill(kb + j, j);
    if (n >= NST)
      direct_barrier<kLoads * (NST - 1)>();
    else
      direct_barrier<0>();
    frags(Set0{}, 0);
    if (n >= NST)
      direct_barrier<kLoads * (NST - 2)>();
    else
      direct_barrier<0>();
  }
  if constexpr (kTail) {
    const int k0 = (tail ? nfull : nfull - 1) * BK, kl = tail ? p.K - nfull * BK : BK;
    tail_a.template load_tail<true, (GUARD & 1) != 0>(k0, kl);
    tail_b.template load_tail<true, (GUARD & 2) != 0>(k0, kl);
  }

  // steady K-tile (tile kt + NST exists): explicit order, since the compiler
  // cannot place inline assembly among the MFMAs by itself
  constexpr int kLast = (kLoads - 1) * SP;  // the MFMA after which the last load goes
  constexpr int kRest = kMfmas - kLast - 1;  // MFMAs after it, among which the fragment reads go
  constexpr int kReads = KG * Cfg::kFragReads;
  // fragment reads per MFMA: one (the 256 and 128 forms, whose last read or none is left
  // to the scheduler), or as many as it takes to place them all
  constexpr int kPer = kReads <= kRest + 1 ? 1 : (kReads + kRest - 1) / (kRest > 0 ? kRest : 1);
  auto steady = [&](auto set, int kt) {
    constexpr int P = decltype(set)::value;
    const int s = (kt - kb) % NST;
    static_for<kLast + 1>([&](auto mc) {
      constexpr int m = decltype(mc)::value;
      mfma(set, mc);
      if constexpr (m % SP == 0) {
        __builtin_amdgcn_sched_barrier(0);
        load_one(m / SP, kt + NST, s);
        __builtin_amdgcn_sched_barrier(0);
      }
    });
    frags(std::integral_constant<int, P ^ 1>{}, (s + 1) % NST);
    static_for<kRest>([&](auto mc) { mfma(set, std::integral_constant<int, decltype(mc)::value + kLast + 1>{}); });
    if constexpr (kRest > 0) sched_interleave<0, kRest, kPer, kReads, 0, 0>();
    direct_barrier<kLoads * (NST - 2)>();
  };
  auto step = [&](auto set, int kt) {
    constexpr int P = decltype(set)::value;
    const int s = (kt - kb) % NST;
    if (kt + NST < kend) fill(kt + NST, s);
    if (kt + 1 < kend) frags(std::integral_constant<int, P ^ 1>{}, (s + 1) % NST);
    static_for<kMfmas>([&](auto mc) { mfma(set, mc); });
    direct_barrier<0>();
  };
  int kt = kb;
  for (; kt + 1 + NST < kend; kt += 2) {  // tiles kt + NST and kt + NST + 1 are in range
    steady(Set0{}, kt);
    steady(Set1{}, kt + 1);
  }
  for (; kt < kend; kt += 2) {
    step(Set0{}, kt);
    if (kt + 1 < kend) step(Set1{}, kt + 1);
  }
  if constexpr (kTail) {
    if (tail) {  // the stages are free: the last direct_barrier<0> left no read pending
      tail_a.store(a_stage(0));
      tail_b.store(b_stage(0));
      __syncthreads();
      frags(Set0{}, 0);
      // MFMA steps whose k all lie past K are skipped, as in mfma_tile_pf
      const int kl = p.K - nfull * BK, ks_u = __builtin_amdgcn_readfirstlane(ks);
      static_for<kMfmas>([&](auto mc) {
        constexpr int m = decltype(mc)::value, r = m / (8 * FM * FN), e = (m / (FM * FN)) % 8;
        if (16 * (ks_u * KG + r) + e < kl) mfma(Set0{}, mc);
      });
      __syncthreads();  // every wavefront's fragment reads done before finish_acc's writes
    }
  }
  // the last direct_barrier<0> (or the tail's barrier) leaves no load in flight and no
  // fragment read pending, so finish_acc may pass the K-split partials through the stages
  finish_acc<BM, BN, WM, WN, KS, FM, FN, Cfg::VA, Cfg::VB, GUARD>(p, acc, smem, m0, n0, part);
}

}  // namespace mfma_detail
}  // namespace sgemm_impl
