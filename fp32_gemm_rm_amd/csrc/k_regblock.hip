// Register-blocked, double-buffered SGEMM on the vector ALU.
//
// Prior art on the pages: each thread keeps an S x S block of C in registers
// ("GPU-accelerated matrix computation ..." section 3.3, register-cache GEMM);
// the sgemmNN page keeps 16 accumulators per thread, streams operands through
// registers and pads its transposing shared-memory store (bs[16][17]); the
// mhpn.cn page ("GEMM advanced: ILP and bank conflicts") sections 2-3
// double-buffers A (stored K-major) and B tiles in shared memory with one
// barrier per K-step and rearranges which lanes read which fragment.
//
// gfx950 design (256 threads = four 64-lane wavefronts, a 16 x 16 grid of
// threads, each owning TM x TN outputs):
//   - A tile BM x BK is loaded with one 128-bit load per thread (4 consecutive
//     k of one row) and stored transposed into As[k][m] (K-major), so that the
//     inner loop reads a thread's TM rows as float4 / float2 vectors.
//   - B tile BK x BN is loaded with one 128-bit load per thread and stored as is
//     into Bs[k][n].
//   - Row padding of As is chosen for 64 LDS banks of 4 bytes: the 64 lanes of a
//     wavefront store 4 words each, for rows r and K-offsets 4q; the stride SA
//     makes {r + 4q*SA mod 64} distinct across the wavefront, so the
//     transposing store is conflict-free.
//   - A wavefront covers an 8 x 8 block of threads, so every fragment read is 8
//     distinct contiguous vectors, each broadcast to 8 lanes.
//   - Two LDS stages; the global loads of tile t+1 are issued before the FMAs
//     of tile t and stored after them, with a single barrier per tile.
//   - Tiles that reach past M or N and the last tile along K load zeros outside
//     the matrix and store under bounds checks; full tiles take an unchecked
//     path.  This bounds-checked variant on small tiles is also the scalar
//     edge-tile path of the MFMA kernel.
#include "internal.h"

namespace sgemm_impl {
namespace {

template <int V>
struct VecT;
template <>
struct VecT<4> {
  using type = float4;
};
template <>
struct VecT<2> {
  using type = float2;
};

template <int V>
__device__ __forceinline__ void load_vec(float (&dst)[V], const float* src) {
  const typename VecT<V>::type v = *reinterpret_cast<const typename VecT<V>::type*>(src);
  if constexpr (V == 4) {
    dst[0] = v.x; dst[1] = v.y; dst[2] = v.z; dst[3] = v.w;
  } else {
    dst[0] = v.x; dst[1] = v.y;
  }
}

// One float4 of row r, columns c0..c0+3 of a rows x cols matrix; zero outside.
template <bool VEC, bool GUARD>
__device__ __forceinline__ float4 gload4(const float* base, long long ld, int r, int c0, int rows, int cols) {
  if (!GUARD) {
    const float* p = base + (long long)r * ld + c0;
    if (VEC) return *reinterpret_cast<const float4*>(p);
    return make_float4(p[0], p[1], p[2], p[3]);
  }
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  if (r >= rows) return v;
  const float* p = base + (long long)r * ld + c0;
  if (VEC && c0 + 3 < cols) return *reinterpret_cast<const float4*>(p);
  if (c0 + 0 < cols) v.x = p[0];
  if (c0 + 1 < cols) v.y = p[1];
  if (c0 + 2 < cols) v.z = p[2];
  if (c0 + 3 < cols) v.w = p[3];
  return v;
}

template <int BM, int BN, int BK, int TM, int TN>
struct RegBlockCfg {
  static constexpr int kThreads = 256;
  static constexpr int kThrM = BM / TM, kThrN = BN / TN;
  static_assert(kThrM == 16 && kThrN == 16, "16 x 16 thread grid");
  static_assert(BM * BK / 4 == kThreads && BN * BK / 4 == kThreads, "one float4 of A and of B per thread");
  static constexpr int VM = TM >= 4 ? 4 : TM, VN = TN >= 4 ? 4 : TN;  // vector widths of fragments
  static constexpr int GM = TM / VM, GN = TN / VN;                    // fragment groups
  static constexpr int KQ = BK / 4;                                   // float4s per A row
  // A row stride: a wavefront stores 64/KQ consecutive rows for each of KQ K-offsets
  // 4q, so 4*SA mod 64 must equal 64/KQ (32, 16, 8 for BM = 128, 64, 32).
  static constexpr int SA = BM + (BM == 128 ? 8 : BM == 64 ? 4 : 2);
  static constexpr int SB = BN;
};

template <int BM, int BN, int BK, int TM, int TN, bool VEC, bool GUARD>
__device__ __forceinline__ void regblock_tile(const Problem& p, int m0, int n0,
                                              float (*As)[BK][RegBlockCfg<BM, BN, BK, TM, TN>::SA],
                                              float (*Bs)[BK][BN]) {
  using Cfg = RegBlockCfg<BM, BN, BK, TM, TN>;
  const int t = threadIdx.x;
  const int w = t / 64, l = t % 64;
  const int tm = (w / 2) * 8 + l / 8;
  const int tn = (w % 2) * 8 + l % 8;

  // global-load coordinates of this thread's float4 of A and of B
  const int a_row = t / Cfg::KQ, a_k4 = (t % Cfg::KQ) * 4;
  const int b_k = t / (BN / 4), b_n4 = (t % (BN / 4)) * 4;
  const float* Ablk = p.A + (long long)m0 * p.lda;
  const float* Bblk = p.B + n0;
  const int rows_left = p.M - m0, cols_left = p.N - n0;

  float acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = 0.f;

  const int ntiles = (p.K + BK - 1) / BK;
  const bool k_ragged = (p.K % BK) != 0;

  auto load_tile = [&](int kt, float4& av, float4& bv) {
    const int k0 = kt * BK;
    if (GUARD || (k_ragged && kt == ntiles - 1)) {
      av = gload4<VEC, true>(Ablk + k0, p.lda, a_row, a_k4, rows_left, p.K - k0);
      bv = gload4<VEC, true>(Bblk + (long long)k0 * p.ldb, p.ldb, b_k, b_n4, p.K - k0, cols_left);
    } else {
      av = gload4<VEC, false>(Ablk + k0, p.lda, a_row, a_k4, rows_left, p.K - k0);
      bv = gload4<VEC, false>(Bblk + (long long)k0 * p.ldb, p.ldb, b_k, b_n4, p.K - k0, cols_left);
    }
  };
  auto store_tile = [&](int s, const float4& av, const float4& bv) {
    As[s][a_k4 + 0][a_row] = av.x;
    As[s][a_k4 + 1][a_row] = av.y;
    As[s][a_k4 + 2][a_row] = av.z;
    As[s][a_k4 + 3][a_row] = av.w;
    *reinterpret_cast<float4*>(&Bs[s][b_k][b_n4]) = bv;
  };

  float4 av, bv;
  load_tile(0, av, bv);
  store_tile(0, av, bv);
  __syncthreads();

  for (int kt = 0; kt < ntiles; ++kt) {
    const int s = kt & 1;
    const bool more = kt + 1 < ntiles;
    if (more) load_tile(kt + 1, av, bv);
#pragma unroll
    for (int k = 0; k < BK; ++k) {
      float a[TM], b[TN];
#pragma unroll
      for (int g = 0; g < Cfg::GM; ++g)
        load_vec<Cfg::VM>(*reinterpret_cast<float(*)[Cfg::VM]>(&a[g * Cfg::VM]),
                          &As[s][k][g * (BM / Cfg::GM) + tm * Cfg::VM]);
#pragma unroll
      for (int g = 0; g < Cfg::GN; ++g)
        load_vec<Cfg::VN>(*reinterpret_cast<float(*)[Cfg::VN]>(&b[g * Cfg::VN]),
                          &Bs[s][k][g * (BN / Cfg::GN) + tn * Cfg::VN]);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    if (more) store_tile(s ^ 1, av, bv);
    __syncthreads();
  }

  // epilogue: C = alpha*acc + beta*C, columns past N and rows past M untouched
  const bool beta0 = p.beta == 0.0f;
#pragma unroll
  for (int gi = 0; gi < Cfg::GM; ++gi)
#pragma unroll
    for (int vi = 0; vi < Cfg::VM; ++vi) {
      const int r = gi * (BM / Cfg::GM) + tm * Cfg::VM + vi;
      if (GUARD && r >= rows_left) continue;
      float* crow = p.C + (long long)(m0 + r) * p.ldc + n0;
#pragma unroll
      for (int gj = 0; gj < Cfg::GN; ++gj)
#pragma unroll
        for (int vj = 0; vj < Cfg::VN; ++vj) {
          const int c = gj * (BN / Cfg::GN) + tn * Cfg::VN + vj;
          if (GUARD && c >= cols_left) continue;
          const float x = acc[gi * Cfg::VM + vi][gj * Cfg::VN + vj];
          crow[c] = beta0 ? p.alpha * x : fmaf(p.alpha, x, p.beta * crow[c]);
        }
    }
}

template <int BM, int BN, int BK, int TM, int TN, bool VEC>
__global__ __launch_bounds__(256) void regblock_kernel(Problem p, int col_blocks) {
  __shared__ __attribute__((aligned(16))) float As[2][BK][RegBlockCfg<BM, BN, BK, TM, TN>::SA];
  __shared__ __attribute__((aligned(16))) float Bs[2][BK][BN];
  const int bm = blockIdx.x / col_blocks;
  const int bn = blockIdx.x - bm * col_blocks;
  const int m0 = bm * BM, n0 = bn * BN;
  if (m0 + BM <= p.M && n0 + BN <= p.N)
    regblock_tile<BM, BN, BK, TM, TN, VEC, false>(p, m0, n0, As, Bs);
  else
    regblock_tile<BM, BN, BK, TM, TN, VEC, true>(p, m0, n0, As, Bs);
}

template <int BM, int BN, int BK, int TM, int TN>
hipError_t launch_cfg(const Problem& p, hipStream_t stream) {
  const long long cb = (p.N + BN - 1) / BN;
  const long long rb = (p.M + BM - 1) / BM;
  if (cb * rb > kMaxGrid) return hipErrorInvalidConfiguration;
  const bool vec = vec4_ok(p.A, p.lda) && vec4_ok(p.B, p.ldb);
  if (vec)
    hipLaunchKernelGGL((regblock_kernel<BM, BN, BK, TM, TN, true>), dim3((unsigned)(cb * rb)), dim3(256), 0,
                       stream, p, (int)cb);
  else
    hipLaunchKernelGGL((regblock_kernel<BM, BN, BK, TM, TN, false>), dim3((unsigned)(cb * rb)), dim3(256), 0,
                       stream, p, (int)cb);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_regblock(const Problem& p, hipStream_t stream) {
  // 128 x 128 tiles when they fill the chip, else 64 x 64.
  const long long tiles128 = (long long)((p.M + 127) / 128) * ((p.N + 127) / 128);
  if (tiles128 >= 512) return launch_cfg<128, 128, 8, 8, 8>(p, stream);
  return launch_cfg<64, 64, 16, 4, 4>(p, stream);
}

hipError_t launch_edge(const Problem& p, hipStream_t stream) {
  return launch_cfg<32, 32, 32, 2, 2>(p, stream);
}

}  // namespace sgemm_impl
