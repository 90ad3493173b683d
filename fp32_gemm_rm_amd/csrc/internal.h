// Internal declarations shared by the kernels and the dispatcher of libsgemm_rm.
// Device code here targets gfx950 only (64-lane wavefronts, 160 KiB LDS per CU,
// FP32 MFMA).  Nothing in this directory is shared with the CPU oracle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sgemm_impl {

// One GEMM problem as the kernels see it.  Leading dimensions are 64-bit so that
// every offset i*ld + j is computed without 32-bit overflow.
struct Problem {
  int M, N, K;
  float alpha, beta;
  const float* A;
  long long lda;
  const float* B;
  long long ldb;
  float* C;
  long long ldc;
  // strided batch: matrix b of the batch starts at A + b*sA, B + b*sB, C + b*sC;
  // the batch index is blockIdx.y (0 for a single GEMM)
  long long sA, sB, sC;
  // op(A) = A^T (A stored K x M, element (m, k) at A[k*lda + m]) / op(B) = B^T (B stored
  // N x K, element (k, n) at B[n*ldb + k]); C is always the M x N row-major result
  int ta, tb;
};

// The problem of batch entry blockIdx.y (device side, at the top of every kernel).
__device__ __forceinline__ Problem batch_entry(Problem p) {
  const long long b = blockIdx.y;
  p.A += b * p.sA;
  p.B += b * p.sB;
  p.C += b * p.sC;
  return p;
}

// Sub-problem covering rows [m0, m0+rows) and columns [n0, n0+cols) of C: the same
// leading dimensions and batch strides, the operands moved to row m0 of op(A) (a
// column offset when A is stored transposed) and column n0 of op(B) (a row offset
// when B is).
inline Problem sub_problem(const Problem& p, int m0, int n0, int rows, int cols) {
  Problem q = p;
  q.M = rows;
  q.N = cols;
  q.A = p.A + (p.ta ? (long long)m0 : (long long)m0 * p.lda);
  q.B = p.B + (p.tb ? (long long)n0 * p.ldb : (long long)n0);
  q.C = p.C + (long long)m0 * p.ldc + n0;
  return q;
}

// True when 128-bit loads along rows of X (base pointer x, leading dimension ld)
// stay 16-byte aligned: the base is 16-byte aligned and ld is a multiple of 4.
inline bool vec4_ok(const void* x, long long ld) {
  return ((uintptr_t)x % 16 == 0) && (ld % 4 == 0);
}

// True when every entry of a batch of `batch` problems may take 128-bit loads of A and
// B: entry b reads from A + b*sA and B + b*sB, so past the first entry the batch strides
// must keep the 16-byte alignment too.
inline bool vec_loads_ok(const Problem& p, int batch) {
  return vec4_ok(p.A, p.lda) && vec4_ok(p.B, p.ldb) && (batch <= 1 || (p.sA % 4 == 0 && p.sB % 4 == 0));
}

// Whether the direct K loop (mfma_direct.h, LDS-DMA loads) of the configuration with
// R x R tiles and K-tiles of BK can load this problem: 16-byte aligned rows
// (vec_loads_ok), whole K-tiles (K a multiple of BK: a partial one would need zeros past
// K, which the LDS-DMA loads cannot write; loaded through registers beside them, it made
// the 256 configuration's kernel spill) unless `tail` (the 64 configuration loads its
// partial last K-tile through registers), and every byte offset from a K-tile's origin
// below 2^31 (the buffer offsets are 32-bit).
inline bool direct_ok(const Problem& p, int batch, int R = 256, int BK = 16, bool tail = false) {
  if (!vec_loads_ok(p, batch) || (!tail && p.K % BK != 0)) return false;
  constexpr long long kLimit = 1LL << 31;
  const long long a = p.ta ? (BK - 1LL) * p.lda + R : (R - 1LL) * p.lda + BK;  // floats past the origin
  const long long b = p.tb ? (R - 1LL) * p.ldb + BK : (BK - 1LL) * p.ldb + R;
  return a * 4 < kLimit && b * 4 < kLimit;
}

// The configurations whose direct K loop runs a problem and is priced apart (tile_plan.h),
// one bit per tile side: the 256 and 128 configurations (BK 16) and the 64 one (BK 32),
// wherever direct_ok allows it.  The 192 configuration's launcher checks direct_ok itself:
// there the direct loop costs what the register-staged one does.
enum : int { kDirect256 = 1, kDirect128 = 2, kDirect64 = 4 };
inline int direct_mask(const Problem& p, int batch) {
  return (direct_ok(p, batch) ? kDirect256 : 0) | (direct_ok(p, batch, 128) ? kDirect128 : 0) |
         (direct_ok(p, batch, 64, 32, true) ? kDirect64 : 0);
}

// Launchers.  Each enqueues its kernel(s) on `stream` and returns the launch status.
// Every launcher accepts any M, N >= 1 and K >= 1 and any leading dimensions, and runs
// `batch` (1 .. kMaxBatch) problems spaced by p.sA, p.sB, p.sC as grid dimension y.
hipError_t launch_naive(const Problem& p, int batch, hipStream_t stream);
hipError_t launch_lds_tiled(const Problem& p, int batch, hipStream_t stream);
hipError_t launch_regblock(const Problem& p, int batch, hipStream_t stream);
// MFMA tiles for the full BM x BN tiles plus bounds-checked register-blocked
// tiles (the scalar edge-tile path) for the strips past them, in one launch; one
// instantiation per operand orientation (p.ta, p.tb), dispatched by launch_mfma.
// tiles: the tile configuration by its side (256, 192, 128, 64, 32 or 16; see tile_plan.h).
// ws: nullptr, or kStreamKBytes of device memory for stream-K (256 configuration, batch 1)
// or for the K slices of the 64 configuration (slices > 1, batch 1; k_slices).
hipError_t launch_mfma_nn(const Problem& p, int batch, hipStream_t stream, int tiles, float* ws, int slices);
hipError_t launch_mfma_nt(const Problem& p, int batch, hipStream_t stream, int tiles, float* ws, int slices);
hipError_t launch_mfma_tn(const Problem& p, int batch, hipStream_t stream, int tiles, float* ws, int slices);
hipError_t launch_mfma_tt(const Problem& p, int batch, hipStream_t stream, int tiles, float* ws, int slices);
inline hipError_t launch_mfma(const Problem& p, int batch, hipStream_t stream, int tiles, float* ws = nullptr,
                              int slices = 1) {
  if (p.ta)
    return p.tb ? launch_mfma_tt(p, batch, stream, tiles, ws, slices)
                : launch_mfma_tn(p, batch, stream, tiles, ws, slices);
  return p.tb ? launch_mfma_nt(p, batch, stream, tiles, ws, slices)
              : launch_mfma_nn(p, batch, stream, tiles, ws, slices);
}

// Compute units of an MI355X (8 XCDs of 32).
constexpr int kCUs = 256;
// Stream-K for the 256 x 256 configuration: the workgroups that share the last waves of
// tiles (one per CU), and the workspace their partial tiles need (two 256 x 256 slots
// each, 128 MiB).
constexpr int kStreamKWgs = kCUs;
constexpr long long kStreamKBytes = 2LL * kStreamKWgs * 256 * 256 * 4;
// Partial MFMA tiles.  A strip of rows (columns) past the last full tile that is at least
// mfma_edge_min(side) wide runs as guarded MFMA tiles of the same grid; a thinner one runs
// as thin strips (192, 128 and 64 configurations: 16, below which a strip would pay for a
// whole tile row or column of MFMA work; 32 configuration: 4) or, in the 256 configuration
// on the register-staged loop (0: never MFMA), as scalar edge tiles (its workgroups fill a
// CU's register file; the cost model steers ragged shapes to the smaller configurations);
// in the 16 configuration every block is guarded (1).  The 256 configuration's direct K
// loop (direct_ok) runs guarded tiles down to kThin256 and thin strips below it.
constexpr int mfma_edge_min(int side) { return side == 256 ? 0 : side == 32 ? 4 : side == 16 ? 1 : 16; }
// The 256 configuration's thin-strip form on the register-staged loop: where both
// remainders past its full tiles are thinner than kThin256, they run as thin strips (same
// launch, after the tiles) instead of scalar edge tiles.  On the direct loop it is also
// the narrowest guarded tile.
constexpr int kThin256 = 16;
constexpr bool thin256(int M, int N) { return M % 256 < kThin256 && N % 256 < kThin256; }
// The extent [0, result) of rows (columns) that MFMA tiles of this side cover, out of n.
constexpr int mfma_extent(int n, int side, int edge_min) {
  return (edge_min > 0 && n % side >= edge_min) ? n : n - n % side;
}

// C := beta*C on the M x N window (zeros when beta == 0; C is then not read).
hipError_t launch_scale(const Problem& p, int batch, hipStream_t stream);

// Largest grid the launchers use: x counts tiles, y counts batch entries.  A dispatch
// counts its work-items per dimension in 32 bits, so blocks times threads per block
// along x must stay below 2^32 as well (grid_fits).
constexpr long long kMaxGrid = 0x7fffffffLL;
constexpr long long kMaxWorkItems = 0xffffffffLL;
constexpr int kMaxBatch = 65535;
inline bool grid_fits(long long blocks, int threads) {
  return blocks <= kMaxGrid && blocks * threads <= kMaxWorkItems;
}
// The one-thread-per-element kernels (naive, scale) cap their grid at this many blocks and
// stride over the rest, so that any M x N fits one launch.
constexpr long long kStrideBlocks = 1LL << 20;
// Largest output window one tiled launch covers.  No tiled launch runs more than 32
// threads per row of C and 16 of its columns (the 16 configuration: a 512-thread workgroup
// per 16 x 16 block; the other configurations, the thin strips and the edge tiles run
// fewer, also on windows narrower than their tiles), so a launch over R rows and C columns
// has at most 32 ceil16(R) ceil(C / 16) work-items.  A window where that product could
// pass 2^32 - 1 runs as bands of rows (and of columns, for rows wider than
// kBandUnits / kBandAlign units of 16), each band a launch of its own on the same stream.
// Band edges fall on multiples of kBandAlign, a multiple of every tile side (256, 192,
// 128, 64, 32, 16), so each band sees whole tiles where the window has them.
constexpr long long kBandUnits = (1LL << 27) - 1;  // ceil16(R) x ceil(C / 16) per launch
constexpr int kBandAlign = 768;
inline bool needs_bands(long long M, long long N) { return (M + 15) / 16 * 16 * ((N + 15) / 16) > kBandUnits; }
// Rows bm and columns bn of the bands of an M x N window (the last band of a row or column
// may be smaller).
inline void band_shape(long long M, long long N, int& bm, int& bn) {
  const long long units = (N + 15) / 16, max_units = kBandUnits / kBandAlign;
  const long long cols = units <= max_units ? N : max_units * 16 / kBandAlign * kBandAlign;
  const long long rows = kBandUnits / ((cols + 15) / 16) / kBandAlign * kBandAlign;  // >= kBandAlign
  bm = (int)(rows < M ? rows : M);
  bn = (int)cols;
}

// Debug build (-DSGEMM_RM_POISON_LDS=1, built as libsgemm_rm_poison.so): every kernel that
// uses LDS fills it with NaN before anything else, so that a read of LDS that no thread of
// the launch has written (a missing barrier, a part of a tile left unfilled) turns into
// NaN in C instead of reading whatever an earlier launch left there.  The production
// build compiles this to nothing.
#ifndef SGEMM_RM_POISON_LDS
#define SGEMM_RM_POISON_LDS 0
#endif
__device__ __forceinline__ void poison_lds(float* p, int n) {
  if constexpr (SGEMM_RM_POISON_LDS != 0) {
    for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = __builtin_nanf("");
    __syncthreads();
  }
}

}  // namespace sgemm_impl
