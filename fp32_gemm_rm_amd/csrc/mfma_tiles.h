// MFMA SGEMM, the two K-loop pipelines of one output tile: mfma_tile (fragments read
// at each k-group) and mfma_tile_pf (fragments read one K-tile ahead, memory
// instructions interleaved with the MFMAs by scheduling-group barriers).
#pragma once

#include <type_traits>
#include "mfma_epilogue.h"
#include "mfma_strips.h"

namespace sgemm_impl {
namespace mfma_detail {

// K-tiles [kb, ke) of the BM x BN tile of C at (m0, n0).  part == nullptr: the range is
// the whole K range and the result goes to C (alpha, beta); otherwise the raw sums go to
// part, a BM x BN row-major block (a stream-K partial tile).  GUARD bit 0 (1): the tile
// reaches past M, bit 1 (2): past N (loads stay inside the matrix, stores skip what is
// past it); bit 2 (4): the launch holds full tiles only (the epilogue's choice of C
// stores).
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
      read_frags<OpA, FM, Cfg::VA>(a_stage(s), wm0, g, lr, lh, af);
      read_frags<OpB, FN, Cfg::VB>(b_stage(s), wn0, g, lr, lh, bf);
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

  finish_acc<BM, BN, WM, WN, KS, FM, FN, Cfg::VA, Cfg::VB, GUARD>(p, acc, smem, m0, n0, part);
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
// KG 16-deep k-groups per wavefront and K-tile (BK = 16 KS KG; the fragments of a K-tile
// take 2 KG (FM + FN) 8 registers per lane).  The MFMA fragments are read
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
//   arrive: one in the 192 configuration (72 MFMAs per wavefront and K-tile; a second
//   set measured no better), two in the 256, 128 and 64 configurations (128, 32 and 8;
//   in the 256 one the second set fits beside the 128 fragment registers once B's
//   fragments are read as 128-bit vectors).
//   FUSE: the tile also computes rows [srow0, srow0 + srows) of a right thin strip,
//   columns [sn0, sn0 + sw) (FusedStrip): its loads, LDS stores and operand reads ride with
//   the tile's, and its FMAs run during the MFMAs of the next K-tile.
template <int BM, int BN, int BK, int WM, int WN, int KS, int NSETS, bool TA, bool TB, bool VEC, int GUARD,
          bool FUSE = false>
__device__ __forceinline__ void mfma_tile_pf(const Problem& p, int m0, int n0, int kb, int ke, float* smem,
                                             float* part = nullptr, int srow0 = 0, int srows = 0, int sn0 = 0,
                                             int sw = 0) {
  using Cfg = MfmaCfg<BM, BN, BK, WM, WN, KS, TA, TB>;
  using OpA = typename Cfg::OpA;
  using OpB = typename Cfg::OpB;
  constexpr int FM = Cfg::FM, FN = Cfg::FN, KG = Cfg::KG;
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
  using FS = FusedStrip<BK, Cfg::kThreads>;
  static_assert(!FUSE || (!TA && !TB && KG == 1), "fused strips: A along k, B along n, one k-group per K-tile");
  static_assert(!FUSE || KS > 1, "fused strips: finish_acc's K-split barrier orders the strip's sums");
  static_assert(!FUSE || KS * WM * WN * FM * FN * 16 * 64 <= 2 * Cfg::kStageFloats,
                "fused strips: finish_acc's K-split partials lie below the strip's stages");
  FS fs;
  if constexpr (FUSE) fs.init(p, sn0, sw, t);
  // the strip's B stages follow the tile's two stages; its A row (clamped where the tile
  // holds no strip rows)
  auto s_stage = [&](int s) { return smem + 2 * Cfg::kStageFloats + s * FS::kStageFloats; };
  const int srow = FUSE ? min(srow0 - m0 + fs.i, BM - 1) : 0;

  v16f acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  float af[2][KG][FM][8], bf[2][KG][FN][8];

  const int nfull = p.K / BK;
  auto load = [&](auto set, int kt) {
    constexpr int R = decltype(set)::value % NSETS;
    if (kt < nfull) {
      opa.template load_full<VEC, GA, R>(kt * BK);
      opb.template load_full<VEC, GB, R>(kt * BK);
      if constexpr (FUSE) fs.template load_full<R>(kt * BK);
    } else {
      opa.template load_tail<VEC, GA, R>(kt * BK, p.K - kt * BK);
      opb.template load_tail<VEC, GB, R>(kt * BK, p.K - kt * BK);
      if constexpr (FUSE) fs.template load_tail<R>(kt * BK, p.K - kt * BK);
    }
  };
  // K-tile kt's global registers to LDS stage s (FULL: kt is a full K-tile)
  auto store = [&](auto set, int s, int kt, auto full) {
    constexpr int R = decltype(set)::value % NSETS;
    opa.template store<R>(a_stage(s));
    opb.template store<R>(b_stage(s));
    if constexpr (FUSE) {
      if constexpr (decltype(full)::value)
        fs.template store<R>(s_stage(s));
      else
        fs.template store<R>(s_stage(s), p.K - kt * BK);
    }
  };
  auto frags = [&](auto set, int s) {
    constexpr int S = decltype(set)::value;
#pragma unroll
    for (int r = 0; r < KG; ++r) {
      read_frags<OpA, FM, Cfg::VA>(a_stage(s), wm0, ks * KG + r, lr, lh, af[S][r]);
      read_frags<OpB, FN, Cfg::VB>(b_stage(s), wn0, ks * KG + r, lr, lh, bf[S][r]);
    }
    if constexpr (FUSE) fs.template read<S>(a_stage(s), s_stage(s), srow);
  };
  const int ks_u = __builtin_amdgcn_readfirstlane(ks);  // K-group, as a uniform value
  // kl: the K-tile's valid k (BK: a full one).  MFMA step e of k-group g takes k = 16g + e
  // and 16g + 8 + e; where both lie past K their operands are zeros, and the step is
  // skipped (adding +0 products to an accumulator that starts at +0 changes no bit).
  auto mfmas = [&](auto set, int kl = BK) {
    constexpr int S = decltype(set)::value;
    if constexpr (FUSE) fs.template fma<S>();
#pragma unroll
    for (int r = 0; r < KG; ++r)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (kl >= BK || 16 * (ks_u * KG + r) + e < kl)
#pragma unroll
          for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[S][r][i][e], bf[S][r][j][e], acc[i][j], 0, 0, 0);
  };
  using Set0 = std::integral_constant<int, 0>;
  using Set1 = std::integral_constant<int, 1>;
  constexpr int D = 2 + NSETS;  // load distance in K-tiles, counted from the tile being multiplied

  // prologue: stage 0 <- tile kb (read into fragment set 0), stage 1 <- tile kb+1, global
  // registers <- tiles kb+2 .. kb+D-1.  FULL: tiles kb .. kb+D+1 exist and are full, and the
  // loads are unconditional: the steady loop's entry then leaves exactly the loads that its
  // back edge leaves in flight, so the compiler's wait before each LDS store covers only
  // the older register set (merged with a prologue whose loads may be skipped, it waits on
  // some of the newest loads too).
  auto prologue = [&](auto full) {
    constexpr bool FULL = decltype(full)::value;
    auto ld = [&](auto set, int kt) {
      if constexpr (FULL) {
        constexpr int R = decltype(set)::value % NSETS;
        opa.template load_full<VEC, GA, R>(kt * BK);
        opb.template load_full<VEC, GB, R>(kt * BK);
        if constexpr (FUSE) fs.template load_full<R>(kt * BK);
      } else if (kt < ke) {
        load(set, kt);
      }
    };
    ld(Set0{}, kb);
    if constexpr (NSETS == 2) ld(Set1{}, kb + 1);
    store(Set0{}, 0, kb, full);
    if constexpr (NSETS == 1)
      ld(Set1{}, kb + 1);
    else
      ld(Set0{}, kb + 2);
    __syncthreads();
    frags(Set0{}, 0);
    if (FULL || kb + 1 < ke) store(Set1{}, 1, kb + 1, full);
    ld(std::integral_constant<int, D - 1>{}, kb + D - 1);
    __syncthreads();
  };

  // Instruction order of a steady K-tile: the MFMAs start right after the barrier and
  // each of the first ones is followed by its share of the memory instructions (LDS
  // stores, then global loads, then fragment reads), so that the wavefronts issue their
  // memory traffic in the shadow of the MFMAs; nothing moves across the barrier (the
  // compiler would otherwise hoist the barrier, and its wait on the fragment reads, above
  // the MFMAs).
  constexpr int kStores = OpA::LOADS + OpB::LOADS + (FUSE ? 1 : 0);
  constexpr int kLoads = OpA::kLoadInstrs(VEC) + OpB::kLoadInstrs(VEC) + (FUSE ? 1 : 0);
  constexpr int kMfmas = 8 * KG * FM * FN;
  constexpr int kMemOps = kStores + kLoads + KG * Cfg::kFragReads + (FUSE ? 2 * FS::SK / 4 : 0);
  constexpr int kPer = (kMemOps + kMfmas - 1) / kMfmas;
  auto steady = [&](auto set, int kt) {  // tiles kt+1 .. kt+D exist and kt+D is full
    constexpr int P = decltype(set)::value;
    __builtin_amdgcn_sched_barrier(0);
    store(set, P, kt + 2, std::true_type{});
    opa.template load_full<VEC, GA, P % NSETS>((kt + D) * BK);
    opb.template load_full<VEC, GB, P % NSETS>((kt + D) * BK);
    if constexpr (FUSE) fs.template load_full<P % NSETS>((kt + D) * BK);
    frags(std::integral_constant<int, P ^ 1>{}, P ^ 1);
    mfmas(set);
    sched_interleave<0, kMfmas, kPer, kMemOps, kStores, kLoads>();
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
  };
  auto step = [&](auto set, int kt) {
    constexpr int P = decltype(set)::value;
    if (kt + 2 < ke) store(set, P, kt + 2, std::false_type{});
    if (kt + D < ke) load(set, kt + D);
    if (kt + 1 < ke) frags(std::integral_constant<int, P ^ 1>{}, P ^ 1);
    mfmas(set, kt < nfull ? BK : p.K - kt * BK);
    __syncthreads();
  };
  int kt = kb;
  const int steady_end = min(ke, nfull);
  auto steady_loop = [&] {
    for (; kt + D + 1 < steady_end; kt += 2) {  // tiles kt+D and kt+D+1 are full and in range
      steady(Set0{}, kt);
      steady(Set1{}, kt + 1);
    }
  };
  if constexpr (BM < 128) {
    // 8 MFMAs per wavefront and K-tile: the one general prologue measured 1-2% faster
    // (1024 x 1024 x 4096: 67.5 against 68.5 us)
    prologue(std::false_type{});
    steady_loop();
  } else if (kb + D + 1 < steady_end) {
    prologue(std::true_type{});
    steady_loop();
  } else {
    prologue(std::false_type{});
  }
  for (; kt < ke; kt += 2) {
    step(Set0{}, kt);
    if (kt + 1 < ke) step(Set1{}, kt + 1);
  }
  // The strip's slice sums go to its first LDS stage (free: the K loop's last fragment
  // reads precede its last barrier, and finish_acc's K-split partials lie below it), and
  // finish_acc's barrier orders them before they are added: a barrier of their own after
  // the tile's C stores would make every wavefront wait for those stores to complete.
  if constexpr (FUSE) {
    fs.load_c(p, srow0, srows, sn0, sw, t);
    fs.stash(s_stage(0), t);
  }
  finish_acc<BM, BN, WM, WN, KS, FM, FN, Cfg::VA, Cfg::VB, GUARD>(p, acc, smem, m0, n0, part);
  if constexpr (FUSE) fs.finish(p, s_stage(0), srow0, srows, sn0, sw, t);
}

}  // namespace mfma_detail
}  // namespace sgemm_impl
