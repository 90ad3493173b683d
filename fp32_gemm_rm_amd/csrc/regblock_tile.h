// Register-blocked, double-buffered SGEMM tile on the vector ALU (device code).
//
// Prior art on the pages: each thread keeps an S x S block of C in registers
// ("GPU-accelerated matrix computation ..." section 3.3, register-cache GEMM);
// the sgemmNN page keeps 16 accumulators per thread, streams operands through
// registers and pads its transposing shared-memory store (bs[16][17]); the
// mhpn.cn page ("GEMM advanced: ILP and bank conflicts") sections 2-3
// double-buffers A (stored K-major) and B tiles in shared memory with one
// barrier per K-step and rearranges which lanes read which fragment.
//
// gfx950 design: NT threads form a (BM/TM) x (BN/TN) grid; each owns TM x TN
// outputs.  Every 64-lane wavefront covers an 8 x 8 block of that grid, so each
// fragment read is 8 distinct contiguous vectors, each broadcast to 8 lanes.
//   - The A tile BM x BK is loaded with one 128-bit load per thread (4
//     consecutive k of one row) and stored transposed into As[k][m] (K-major),
//     so that the inner loop reads a thread's TM rows as float4 / float2.
//   - The B tile BK x BN is loaded with one 128-bit load per thread and stored
//     as is into Bs[k][n].
//   - Transposed operands (A stored K x M, B stored N x K) load along their own
//     contiguous dimension and land in the same As[k][m] / Bs[k][n] layout: A^T
//     rows store straight, B^T rows store transposed.
//   - As rows are padded by PAD_A words.  A wavefront's transposing store
//     writes 64/KQ consecutive rows at each of KQ = BK/4 K-offsets 4q; 32-bit
//     LDS accesses are served per half-wavefront from 32 banks, so the padding
//     is chosen to spread {row + 4q*(BM + PAD_A)} over distinct banks.
//   - Two LDS stages; the global loads of tile t+1 are issued before the FMAs
//     of tile t and stored after them, with a single barrier per tile.
//   - UNROLL bounds how many k-steps of fragment reads the compiler may hoist,
//     which bounds the registers the tile needs.
//   - Loads outside M, N or K read zeros and stores outside M x N are skipped
//     when GUARD is set (tiles that reach past the matrix, and the last K-tile
//     of every tile when K is not a multiple of BK).
//   - compute() may cover a sub-range of K, so that several thread groups can
//     share one tile's K range and add their partial sums (the edge tiles of
//     the MFMA kernel do).
#pragma once

#include "internal.h"

namespace sgemm_impl {

template <int BM, int BN, int BK, int TM, int TN, int NT, int PAD_A, int UNROLL = BK>
struct RegBlock {
  static constexpr int kThrM = BM / TM, kThrN = BN / TN;
  static_assert(kThrM * kThrN == NT, "thread grid covers the tile");
  static_assert(kThrM % 8 == 0 && kThrN % 8 == 0, "8 x 8 threads per wavefront");
  static_assert(BM * BK / 4 == NT && BN * BK / 4 == NT, "one float4 of A and of B per thread");
  static constexpr int VM = TM >= 4 ? 4 : TM, VN = TN >= 4 ? 4 : TN;  // fragment vector widths
  static constexpr int GM = TM / VM, GN = TN / VN;                    // fragment groups
  static constexpr int KQ = BK / 4;
  static_assert(KQ <= NT && BM / 4 <= NT && BN / 4 <= NT, "load coordinates");
  static constexpr int SA = BM + PAD_A;
  static_assert((SA * 4) % (VM * 4) == 0, "fragment reads stay aligned");
  static constexpr int kLdsFloats = 2 * BK * SA + 2 * BK * BN;  // two stages of As and Bs

  template <int V>
  static __device__ __forceinline__ void read_vec(float* dst, const float* src) {
    if constexpr (V == 4) {
      const float4 v = *reinterpret_cast<const float4*>(src);
      dst[0] = v.x; dst[1] = v.y; dst[2] = v.z; dst[3] = v.w;
    } else if constexpr (V == 2) {
      const float2 v = *reinterpret_cast<const float2*>(src);
      dst[0] = v.x; dst[1] = v.y;
    } else {
      dst[0] = src[0];
    }
  }

  // One float4 of row r, columns c0..c0+3 of a rows x cols matrix; zero outside when checked.
  template <bool VEC, bool CHECK>
  static __device__ __forceinline__ float4 gload4(const float* base, long long ld, int r, int c0, int rows,
                                                  int cols) {
    if (!CHECK) {
      const float* q = base + (long long)r * ld + c0;
      if (VEC) return *reinterpret_cast<const float4*>(q);
      return make_float4(q[0], q[1], q[2], q[3]);
    }
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (r >= rows) return v;
    const float* q = base + (long long)r * ld + c0;
    if (VEC && c0 + 3 < cols) return *reinterpret_cast<const float4*>(q);
    if (c0 + 0 < cols) v.x = q[0];
    if (c0 + 1 < cols) v.y = q[1];
    if (c0 + 2 < cols) v.z = q[2];
    if (c0 + 3 < cols) v.w = q[3];
    return v;
  }

  // acc = op(A)[m0.., kbeg : kbeg+klen] op(B)[kbeg : kbeg+klen, n0..] for one BM x BN tile,
  // in `ntiles` K-steps of BK (ntiles * BK >= klen; every thread of the workgroup must pass
  // the same ntiles, since each K-step ends with a workgroup barrier).  TA / TB: A is
  // stored K x M (element (m, k) at A[k*lda + m]) / B is stored N x K.  lds points to
  // kLdsFloats floats of 16-byte aligned LDS; tid in [0, NT).
  template <bool VEC, bool GUARD, bool TA = false, bool TB = false>
  static __device__ __forceinline__ void compute(const Problem& p, int m0, int n0, int kbeg, int klen, int ntiles,
                                                 float* lds, int tid, float (&acc)[TM][TN]) {
    float* As = lds;                 // [2][BK][SA]
    float* Bs = lds + 2 * BK * SA;   // [2][BK][BN]
    const int w = tid / 64, l = tid % 64;
    constexpr int WAVES_N = kThrN / 8;
    const int tm = (w / WAVES_N) * 8 + l / 8;
    const int tn = (w % WAVES_N) * 8 + l % 8;

    // one float4 of A and one of B per thread and K-step, along the operand's contiguous
    // dimension: A rows of k (A untransposed) or rows of m (transposed), likewise for B
    const int a_r = TA ? tid / (BM / 4) : tid / KQ;
    const int a_c = TA ? (tid % (BM / 4)) * 4 : (tid % KQ) * 4;
    const int b_r = TB ? tid / KQ : tid / (BN / 4);
    const int b_c = TB ? (tid % KQ) * 4 : (tid % (BN / 4)) * 4;
    const float* Ablk = TA ? p.A + (long long)kbeg * p.lda + m0 : p.A + (long long)m0 * p.lda + kbeg;
    const float* Bblk = TB ? p.B + (long long)n0 * p.ldb + kbeg : p.B + (long long)kbeg * p.ldb + n0;
    const int rows_left = p.M - m0, cols_left = p.N - n0;

#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = 0.f;

    const int nfull = klen / BK;
    float4 av, bv;
    auto load_tile = [&](int kt) {
      const int k0 = kt * BK;
      const float* ap = TA ? Ablk + (long long)k0 * p.lda : Ablk + k0;
      const float* bp = TB ? Bblk + k0 : Bblk + (long long)k0 * p.ldb;
      const int a_rows = TA ? klen - k0 : rows_left, a_cols = TA ? rows_left : klen - k0;
      const int b_rows = TB ? cols_left : klen - k0, b_cols = TB ? klen - k0 : cols_left;
      if (GUARD || kt >= nfull) {
        av = gload4<VEC, true>(ap, p.lda, a_r, a_c, a_rows, a_cols);
        bv = gload4<VEC, true>(bp, p.ldb, b_r, b_c, b_rows, b_cols);
      } else {
        av = gload4<VEC, false>(ap, p.lda, a_r, a_c, a_rows, a_cols);
        bv = gload4<VEC, false>(bp, p.ldb, b_r, b_c, b_rows, b_cols);
      }
    };
    // LDS holds A as As[k][m] and B as Bs[k][n] in every case
    auto store_tile = [&](int s) {
      float* as = As + s * BK * SA;
      float* bs = Bs + s * BK * BN;
      if (TA) {
        as[a_r * SA + a_c + 0] = av.x;
        as[a_r * SA + a_c + 1] = av.y;
        as[a_r * SA + a_c + 2] = av.z;
        as[a_r * SA + a_c + 3] = av.w;
      } else {
        as[(a_c + 0) * SA + a_r] = av.x;
        as[(a_c + 1) * SA + a_r] = av.y;
        as[(a_c + 2) * SA + a_r] = av.z;
        as[(a_c + 3) * SA + a_r] = av.w;
      }
      if (TB) {
        bs[(b_c + 0) * BN + b_r] = bv.x;
        bs[(b_c + 1) * BN + b_r] = bv.y;
        bs[(b_c + 2) * BN + b_r] = bv.z;
        bs[(b_c + 3) * BN + b_r] = bv.w;
      } else {
        *reinterpret_cast<float4*>(bs + b_r * BN + b_c) = bv;
      }
    };

    load_tile(0);
    store_tile(0);
    __syncthreads();
    for (int kt = 0; kt < ntiles; ++kt) {
      const int s = kt & 1;
      const bool more = kt + 1 < ntiles;
      if (more) load_tile(kt + 1);
      const float* as = As + s * BK * SA;
      const float* bs = Bs + s * BK * BN;
#pragma unroll UNROLL
      for (int k = 0; k < BK; ++k) {
        float a[TM], b[TN];
#pragma unroll
        for (int g = 0; g < GM; ++g) read_vec<VM>(&a[g * VM], as + k * SA + g * (BM / GM) + tm * VM);
#pragma unroll
        for (int g = 0; g < GN; ++g) read_vec<VN>(&b[g * VN], bs + k * BN + g * (BN / GN) + tn * VN);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
      }
      if (more) store_tile(s ^ 1);
      __syncthreads();
    }
  }

  // C = alpha*acc + beta*C for the tile; rows past M and columns past N untouched.
  template <bool GUARD>
  static __device__ __forceinline__ void store(const Problem& p, int m0, int n0, int tid,
                                               const float (&acc)[TM][TN]) {
    const int w = tid / 64, l = tid % 64;
    constexpr int WAVES_N = kThrN / 8;
    const int tm = (w / WAVES_N) * 8 + l / 8;
    const int tn = (w % WAVES_N) * 8 + l % 8;
    const int rows_left = p.M - m0, cols_left = p.N - n0;
    // every C value of the thread is loaded before the first store: a load after a store
    // into the same array would wait for that store
    float cin[TM][TN];
    const bool beta0 = p.beta == 0.0f;
#pragma unroll
    for (int pass = beta0 ? 1 : 0; pass < 2; ++pass)
#pragma unroll
      for (int gi = 0; gi < GM; ++gi)
#pragma unroll
        for (int vi = 0; vi < VM; ++vi) {
          const int r = gi * (BM / GM) + tm * VM + vi;
          if (GUARD && r >= rows_left) continue;
          float* crow = p.C + (long long)(m0 + r) * p.ldc + n0;
#pragma unroll
          for (int gj = 0; gj < GN; ++gj)
#pragma unroll
            for (int vj = 0; vj < VN; ++vj) {
              const int c = gj * (BN / GN) + tn * VN + vj;
              if (GUARD && c >= cols_left) continue;
              const int i = gi * VM + vi, j = gj * VN + vj;
              if (pass == 0)
                cin[i][j] = crow[c];
              else
                crow[c] = beta0 ? p.alpha * acc[i][j] : fmaf(p.alpha, acc[i][j], p.beta * cin[i][j]);
            }
        }
  }

  // The whole tile: C[m0.., n0..] = alpha * op(A)[m0.., :] op(B)[:, n0..] + beta * C.
  template <bool VEC, bool GUARD, bool TA = false, bool TB = false>
  static __device__ __forceinline__ void tile(const Problem& p, int m0, int n0, float* lds, int tid) {
    float acc[TM][TN];
    compute<VEC, GUARD, TA, TB>(p, m0, n0, 0, p.K, (p.K + BK - 1) / BK, lds, tid, acc);
    store<GUARD>(p, m0, n0, tid, acc);
  }
};

}  // namespace sgemm_impl
