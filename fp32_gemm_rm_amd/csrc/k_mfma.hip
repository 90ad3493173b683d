// SGEMM on the FP32 matrix cores of gfx950 (v_mfma_f32_32x32x2_f32).
//
// The pages' fastest designs are register-blocked tiles fed from padded,
// double-buffered shared memory (sgemmNN page; mhpn.cn "GEMM advanced" page
// sections 2-3) and, for half precision only, warp-level matrix fragments
// ("GPU-accelerated matrix computation ..." section 2.2).  On gfx950 the dense
// FP32 contraction belongs on the matrix cores, which accept float32 operands
// directly, so this kernel keeps the page's tiling and double buffering and
// replaces the per-thread FMA block with 32 x 32 x 2 MFMA tiles.
//
// MFMA operand layout (32x32x2, checked on the device with one-hot operands):
// lane l supplies A(l%32, kk = l/32) and B(kk = l/32, l%32); accumulator
// register i of lane l holds D(8*(i/4) + 4*(l/32) + i%4, l%32).  Because the
// sum over k may visit k in any order, lane half h = l/32 of one MFMA step e
// takes k = 16g + 8h + e of K-group g (e = 0..7): a lane then reads its eight A
// values for a group as two contiguous 128-bit LDS loads.
//
// Workgroup: WM x WN wavefronts of 64 lanes, macro-tile BM x BN, K-tile BK = 16.
// Each wavefront owns a (BM/WM) x (BN/WN) block of C as (BM/WM/32) x (BN/WN/32)
// accumulators of 16 registers.
//
// LDS (two stages):
//   As[m][k] with row stride 20 words: A tile as loaded (k contiguous), written
//     with 128-bit stores.  A fragment read by lanes 0-15 touches words
//     20r .. 20r+3 for r = 0..15, 64 distinct banks.
//   Bs[k][n] with row stride BN + 4 words: B tile as loaded.  A fragment read
//     is one word per lane: lanes 0-31 read 32 consecutive words of row e and
//     lanes 32-63 the same columns of row 8+e, (8*(BN+4)) mod 64 = 32 banks
//     apart, so the 64 lanes hit 64 distinct banks.
// Global loads are 128-bit (rows 16-byte aligned) or scalar; the last K-tile
// loads zeros past K.  Only full BM x BN tiles run here: the partial tiles along
// M and N go to the scalar edge-tile path.
#include "internal.h"

namespace sgemm_impl {
namespace {

typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int BK = 16;
constexpr int SA = BK + 4;

template <bool VEC, bool GUARD>
__device__ __forceinline__ float4 gload4(const float* p, int c0, int cols) {
  if (!GUARD) {
    if (VEC) return *reinterpret_cast<const float4*>(p);
    return make_float4(p[0], p[1], p[2], p[3]);
  }
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  if (VEC && c0 + 3 < cols) return *reinterpret_cast<const float4*>(p);
  if (c0 + 0 < cols) v.x = p[0];
  if (c0 + 1 < cols) v.y = p[1];
  if (c0 + 2 < cols) v.z = p[2];
  if (c0 + 3 < cols) v.w = p[3];
  return v;
}

template <int BM, int BN, int WM, int WN>
struct MfmaCfg {
  static constexpr int kThreads = WM * WN * 64;
  static constexpr int WTM = BM / WM, WTN = BN / WN;  // wavefront tile
  static constexpr int FM = WTM / 32, FN = WTN / 32;  // 32x32 blocks per wavefront
  static constexpr int SB = BN + 4;
  static constexpr int A_LOADS = BM * BK / 4 / kThreads;  // float4 per thread per K-tile
  static constexpr int B_LOADS = BN * BK / 4 / kThreads;
  static_assert(FM >= 1 && FN >= 1, "wavefront tile at least 32 x 32");
  static_assert(A_LOADS * kThreads * 4 == BM * BK && B_LOADS * kThreads * 4 == BN * BK, "even load split");
};

template <int BM, int BN, int WM, int WN, bool VEC>
__global__ __launch_bounds__(WM* WN * 64) void mfma_kernel(Problem p, int tiles_n) {
  using Cfg = MfmaCfg<BM, BN, WM, WN>;
  constexpr int NT = Cfg::kThreads, FM = Cfg::FM, FN = Cfg::FN, SB = Cfg::SB;
  __shared__ __attribute__((aligned(16))) float As[2][BM][SA];
  __shared__ __attribute__((aligned(16))) float Bs[2][BK][SB];

  const int t = threadIdx.x;
  const int w = t / 64, l = t % 64;
  const int lr = l % 32, lh = l / 32;
  const int wm0 = (w / WN) * Cfg::WTM, wn0 = (w % WN) * Cfg::WTN;

  const int bm = blockIdx.x / tiles_n;
  const int bn = blockIdx.x - bm * tiles_n;
  const int m0 = bm * BM, n0 = bn * BN;
  const float* Ablk = p.A + (long long)m0 * p.lda;
  const float* Bblk = p.B + n0;

  v16f acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int ntiles = (p.K + BK - 1) / BK;
  const bool k_ragged = (p.K % BK) != 0;

  float4 ra[Cfg::A_LOADS], rb[Cfg::B_LOADS];
  auto load_tile = [&](int kt) {
    const int k0 = kt * BK;
    const bool guard = k_ragged && kt == ntiles - 1;
#pragma unroll
    for (int i = 0; i < Cfg::A_LOADS; ++i) {
      const int q = t + i * NT;
      const int row = q / (BK / 4), k4 = (q % (BK / 4)) * 4;
      const float* src = Ablk + (long long)row * p.lda + k0 + k4;
      ra[i] = guard ? gload4<VEC, true>(src, k4, p.K - k0) : gload4<VEC, false>(src, k4, p.K - k0);
    }
#pragma unroll
    for (int i = 0; i < Cfg::B_LOADS; ++i) {
      const int q = t + i * NT;
      const int kr = q / (BN / 4), n4 = (q % (BN / 4)) * 4;
      if (guard && k0 + kr >= p.K) {
        rb[i] = make_float4(0.f, 0.f, 0.f, 0.f);
      } else {
        rb[i] = gload4<VEC, false>(Bblk + (long long)(k0 + kr) * p.ldb + n4, n4, BN);
      }
    }
  };
  auto store_tile = [&](int s) {
#pragma unroll
    for (int i = 0; i < Cfg::A_LOADS; ++i) {
      const int q = t + i * NT;
      const int row = q / (BK / 4), k4 = (q % (BK / 4)) * 4;
      *reinterpret_cast<float4*>(&As[s][row][k4]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < Cfg::B_LOADS; ++i) {
      const int q = t + i * NT;
      const int kr = q / (BN / 4), n4 = (q % (BN / 4)) * 4;
      *reinterpret_cast<float4*>(&Bs[s][kr][n4]) = rb[i];
    }
  };

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int kt = 0; kt < ntiles; ++kt) {
    const int s = kt & 1;
    const bool more = kt + 1 < ntiles;
    if (more) load_tile(kt + 1);

    float af[FM][8], bf[FN][8];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const float4 x0 = *reinterpret_cast<const float4*>(&As[s][wm0 + i * 32 + lr][lh * 8]);
      const float4 x1 = *reinterpret_cast<const float4*>(&As[s][wm0 + i * 32 + lr][lh * 8 + 4]);
      af[i][0] = x0.x; af[i][1] = x0.y; af[i][2] = x0.z; af[i][3] = x0.w;
      af[i][4] = x1.x; af[i][5] = x1.y; af[i][6] = x1.z; af[i][7] = x1.w;
    }
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) bf[j][e] = Bs[s][lh * 8 + e][wn0 + j * 32 + lr];
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[i][e], bf[j][e], acc[i][j], 0, 0, 0);

    if (more) store_tile(s ^ 1);
    __syncthreads();
  }

  // epilogue: register r of lane l is row 8*(r/4) + 4*lh + r%4, column lr of its block
  const bool beta0 = p.beta == 0.0f;
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm0 + i * 32 + 8 * (r / 4) + 4 * lh + (r % 4);
        const int col = n0 + wn0 + j * 32 + lr;
        float* c = p.C + (long long)row * p.ldc + col;
        const float x = acc[i][j][r];
        *c = beta0 ? p.alpha * x : fmaf(p.alpha, x, p.beta * *c);
      }
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_cfg(const Problem& p, hipStream_t stream) {
  const int Mf = (p.M / BM) * BM, Nf = (p.N / BN) * BN;
  if (Mf > 0 && Nf > 0) {
    const long long tn = Nf / BN, tm = Mf / BM;
    if (tn * tm > kMaxGrid) return hipErrorInvalidConfiguration;
    Problem q = sub_problem(p, 0, 0, Mf, Nf);
    const bool vec = vec4_ok(p.A, p.lda) && vec4_ok(p.B, p.ldb);
    if (vec)
      hipLaunchKernelGGL((mfma_kernel<BM, BN, WM, WN, true>), dim3((unsigned)(tn * tm)), dim3(WM * WN * 64), 0,
                         stream, q, (int)tn);
    else
      hipLaunchKernelGGL((mfma_kernel<BM, BN, WM, WN, false>), dim3((unsigned)(tn * tm)), dim3(WM * WN * 64),
                         0, stream, q, (int)tn);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // scalar edge-tile path: columns [Nf, N) of rows [0, Mf), then rows [Mf, M) in full
  if (Mf > 0 && Nf < p.N) {
    hipError_t e = launch_edge(sub_problem(p, 0, Nf, Mf, p.N - Nf), stream);
    if (e != hipSuccess) return e;
  }
  if (Mf < p.M) {
    hipError_t e = launch_edge(sub_problem(p, Mf, 0, p.M - Mf, p.N), stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_mfma(const Problem& p, hipStream_t stream) {
  const long long tiles128 = (long long)(p.M / 128) * (p.N / 128);
  if (tiles128 >= 512) return launch_cfg<128, 128, 2, 2>(p, stream);
  return launch_cfg<64, 64, 2, 2>(p, stream);
}

}  // namespace sgemm_impl
