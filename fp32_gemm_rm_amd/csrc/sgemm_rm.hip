// C-ABI entry points of libsgemm_rm: argument checks, the special cases,
// the choice of kernel family and the launches on the caller's stream.
// The operations and their return codes are specified in include/sgemm_rm.h.
#include "sgemm_rm.h"

#include <cstdint>
#include <mutex>

#include "internal.h"
#include "tile_plan.h"

namespace {

using sgemm_impl::Problem;

// The scratch of sgemm_rm_op_strided_batched_noalloc: the stream-K workspace kept in the
// library's own static device memory, so that the call allocates nothing.  Each GPU the
// library runs on holds its own copy from the code object's load until the process ends.
// In host code `scratch` only names the symbol: its device address, per device, comes
// from hipGetSymbolAddress (scratch_on), and only that address reaches a kernel.
constexpr long long kScratchBytes = SGEMM_RM_SCRATCH_BYTES;
static_assert(kScratchBytes >= sgemm_impl::kStreamKBytes, "the scratch holds a stream-K workspace");
static __device__ __align__(256) float scratch[kScratchBytes / 4];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
float* g_scratch[kMaxDevices];  // device address of `scratch` on each device, once looked up

// The address of `scratch` on the device that `stream` belongs to, looked up on the
// first call for that device with that device current (the caller's current device is
// restored).
hipError_t scratch_on(hipStream_t stream, float** out) {
  hipDevice_t dev = 0;
  hipError_t err = hipStreamGetDevice(stream, &dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch[dev] == nullptr) {
    int cur = 0;
    err = hipGetDevice(&cur);
    if (err != hipSuccess) return err;
    if (cur != dev && (err = hipSetDevice(dev)) != hipSuccess) return err;
    void* ptr = nullptr;
    err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t back = hipSetDevice(cur);
      if (err == hipSuccess) err = back;
    }
    if (err != hipSuccess) return err;
    g_scratch[dev] = static_cast<float*>(ptr);
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

// 1-based positions of the arguments of one entry point; 0 = the entry point has no
// such argument.  Every entry point lists its arguments in this relative order:
// transA transB M N K alpha A lda strideA B ldb strideB beta C ldc strideC batch
// workspace workspace_bytes stream variant.
struct Positions {
  int ta, tb, M, N, K, A, lda, sA, B, ldb, sB, C, ldc, sC, batch, ws, ws_bytes, variant;
};
constexpr Positions kPosRm = {0, 0, 1, 2, 3, 5, 6, 0, 7, 8, 0, 10, 11, 0, 0, 0, 0, 13};
constexpr Positions kPosRmBatched = {0, 0, 1, 2, 3, 5, 6, 7, 8, 9, 10, 12, 13, 14, 15, 0, 0, 17};
constexpr Positions kPosOp = {1, 2, 3, 4, 5, 7, 8, 0, 9, 10, 0, 12, 13, 0, 0, 0, 0, 0};
constexpr Positions kPosOpBatched = {1, 2, 3, 4, 5, 7, 8, 9, 10, 11, 12, 14, 15, 16, 17, 0, 0, 19};
constexpr Positions kPosOpBatchedWs = {1, 2, 3, 4, 5, 7, 8, 9, 10, 11, 12, 14, 15, 16, 17, 18, 19, 21};

// One call in the caller's terms.  cm: column-major storage (element (i, j) of X at
// X[j*ldX + i]); ta / tb: A is stored K x M / B is stored N x K (op = transpose).
struct Call {
  bool cm;
  int ta, tb, M, N, K;
  float alpha;
  const float* A;
  int lda;
  long long sA;
  const float* B;
  int ldb;
  long long sB;
  float beta;
  float* C;
  int ldc;
  long long sC;
  int batch;
  void* ws;  // stream-K workspace (nullptr: none)
  long long ws_bytes;
  int variant;
};

int at_least(int n) { return n > 1 ? n : 1; }

// Argument checks in parameter order; returns 0 or -(position of the first bad one).
int check(const Call& c, const Positions& pos) {
  if (c.ta != 0 && c.ta != 1) return -pos.ta;
  if (c.tb != 0 && c.tb != 1) return -pos.tb;
  if (c.M < 0) return -pos.M;
  if (c.N < 0) return -pos.N;
  if (c.K < 0) return -pos.K;
  const bool any = c.M > 0 && c.N > 0 && c.batch > 0;
  const bool reads_ab = any && c.K > 0 && c.alpha != 0.0f;
  // stored shapes: the leading dimension spans the other index of the storage order
  const int a_rows = c.ta ? c.K : c.M, a_cols = c.ta ? c.M : c.K;
  const int b_rows = c.tb ? c.N : c.K, b_cols = c.tb ? c.K : c.N;
  if (reads_ab && c.A == nullptr) return -pos.A;
  if (c.lda < at_least(c.cm ? a_rows : a_cols)) return -pos.lda;
  if (pos.sA && c.sA < 0) return -pos.sA;
  if (reads_ab && c.B == nullptr) return -pos.B;
  if (c.ldb < at_least(c.cm ? b_rows : b_cols)) return -pos.ldb;
  if (pos.sB && c.sB < 0) return -pos.sB;
  if (any && c.C == nullptr) return -pos.C;
  if (c.ldc < at_least(c.cm ? c.M : c.N)) return -pos.ldc;
  if (pos.sC) {  // the outputs of different batch entries must not overlap
    const long long extent = c.cm ? (long long)(c.N - 1) * c.ldc + c.M : (long long)(c.M - 1) * c.ldc + c.N;
    if (c.sC < 0 || (c.batch > 1 && c.M > 0 && c.N > 0 && c.sC < extent)) return -pos.sC;
  }
  if (pos.batch && c.batch < 0) return -pos.batch;
  if (pos.ws && c.ws == nullptr && c.ws_bytes > 0) return -pos.ws;
  if (pos.ws_bytes && c.ws_bytes < 0) return -pos.ws_bytes;
  if (pos.variant && (c.variant < SGEMM_RM_VARIANT_AUTO || c.variant > SGEMM_RM_VARIANT_MFMA_T16)) return -pos.variant;
  return 0;
}

// Enqueue `batch` problems spaced by p.sA, p.sB, p.sC (p already validated, M, N > 0),
// in launches of at most kMaxBatch entries.  ws: a stream-K workspace of at least
// kStreamKBytes, or nullptr.
int launch_batches(Problem p, int batch, hipStream_t stream, int variant, float* ws) {
  if (batch != 1) ws = nullptr;  // stream-K covers single products only
  while (batch > 0) {
    const int chunk = batch < sgemm_impl::kMaxBatch ? batch : sgemm_impl::kMaxBatch;
    hipError_t err;
    if (p.alpha == 0.0f || p.K == 0) {
      if (p.beta == 1.0f) return 0;
      err = sgemm_impl::launch_scale(p, chunk, stream);
    } else {
      switch (variant) {
        case SGEMM_RM_VARIANT_NAIVE:
          err = sgemm_impl::launch_naive(p, chunk, stream);
          break;
        case SGEMM_RM_VARIANT_LDS_TILED:
          err = sgemm_impl::launch_lds_tiled(p, chunk, stream);
          break;
        case SGEMM_RM_VARIANT_REGBLOCK:
          err = sgemm_impl::launch_regblock(p, chunk, stream);
          break;
        case SGEMM_RM_VARIANT_MFMA_T256:  // with a workspace: stream-K wherever the tiles leave a partial wave
          err = sgemm_impl::launch_mfma(p, chunk, stream, 256, ws);
          break;
        case SGEMM_RM_VARIANT_MFMA_T192:
          err = sgemm_impl::launch_mfma(p, chunk, stream, 192);
          break;
        case SGEMM_RM_VARIANT_MFMA_T128:
          err = sgemm_impl::launch_mfma(p, chunk, stream, 128);
          break;
        case SGEMM_RM_VARIANT_MFMA_T64:  // with a workspace: K slices wherever k_slices applies
          err = sgemm_impl::launch_mfma(p, chunk, stream, 64, ws, sgemm_impl::k_slices(p.M, p.N, p.K, chunk));
          break;
        case SGEMM_RM_VARIANT_MFMA_T32:
          err = sgemm_impl::launch_mfma(p, chunk, stream, 32);
          break;
        case SGEMM_RM_VARIANT_MFMA_T16:
          err = sgemm_impl::launch_mfma(p, chunk, stream, 16);
          break;
        case SGEMM_RM_VARIANT_MFMA:
        case SGEMM_RM_VARIANT_AUTO:
        default: {
          const sgemm_impl::TilePlan plan =
              sgemm_impl::plan_tiles(p.M, p.N, p.K, chunk, ws != nullptr, sgemm_impl::direct_mask(p, chunk));
          err = sgemm_impl::launch_mfma(p, chunk, stream, plan.side, plan.stream_k || plan.slices > 1 ? ws : nullptr,
                                        plan.slices);
          break;
        }
      }
    }
    if (err != hipSuccess) return (int)err;
    batch -= chunk;
    p.A += (long long)chunk * p.sA;
    p.B += (long long)chunk * p.sB;
    p.C += (long long)chunk * p.sC;
  }
  return 0;
}

// As launch_batches, with a C window too large for one tiled launch's 32-bit work-item
// count (needs_bands) cut into bands of rows, and of columns for very long rows
// (band_shape), that launch one after another on the same stream.  The
// one-thread-per-element kernels (naive, and the scale pass of alpha == 0 or K == 0)
// stride over a capped grid and take the window whole.
int launch(const Problem& p, int batch, hipStream_t stream, int variant, float* ws) {
  const bool strided = variant == SGEMM_RM_VARIANT_NAIVE || p.alpha == 0.0f || p.K == 0;
  if (strided || !sgemm_impl::needs_bands(p.M, p.N)) return launch_batches(p, batch, stream, variant, ws);
  int bm, bn;
  sgemm_impl::band_shape(p.M, p.N, bm, bn);
  for (long long m0 = 0; m0 < p.M; m0 += bm)
    for (long long n0 = 0; n0 < p.N; n0 += bn) {
      const int rows_b = (int)(bm < p.M - m0 ? bm : p.M - m0), cols_b = (int)(bn < p.N - n0 ? bn : p.N - n0);
      const int rc = launch_batches(sgemm_impl::sub_problem(p, (int)m0, (int)n0, rows_b, cols_b), batch, stream,
                                    variant, ws);
      if (rc != 0) return rc;
    }
  return 0;
}

// Workspace bytes that a call's kernels may use given a large enough workspace (0: none
// of them can): stream-K or K slices, single products only, where the default path's cost
// model picks them, the 256 configuration is forced (stream-K), the 64 one is forced on a
// shape that K slices apply to, or a banded window (launch) leaves the choice to each band.
// An over-estimate only costs the scratch lookup; the launchers decide.
long long workspace_need(const Problem& p, int batch, int variant) {
  if (batch != 1 || p.alpha == 0.0f || p.K == 0) return 0;
  if (variant == SGEMM_RM_VARIANT_MFMA_T256) return sgemm_impl::kStreamKBytes;
  if (variant == SGEMM_RM_VARIANT_MFMA_T64)
    return sgemm_impl::k_slices(p.M, p.N, p.K, 1) > 1 ? sgemm_impl::kStreamKBytes : 0;
  if (variant != SGEMM_RM_VARIANT_AUTO && variant != SGEMM_RM_VARIANT_MFMA) return 0;
  if (sgemm_impl::needs_bands(p.M, p.N)) return sgemm_impl::kStreamKBytes;
  const sgemm_impl::TilePlan plan = sgemm_impl::plan_tiles(p.M, p.N, p.K, 1, true, sgemm_impl::direct_mask(p, 1));
  return plan.stream_k || plan.slices > 1 ? sgemm_impl::kStreamKBytes : 0;
}

// Validate, then run as a row-major problem.  A column-major product C = op(A) op(B)
// is the row-major product C^T = op(B)^T op(A)^T over the same memory: a column-major
// X is the row-major X^T with the same leading dimension, so the operands and M, N
// swap and each operand keeps its transpose flag.
int run(const Call& c, const Positions& pos, hipStream_t stream, bool use_scratch = false) {
  const int bad = check(c, pos);
  if (bad != 0) return bad;
  if (c.M == 0 || c.N == 0 || c.batch == 0) return 0;
  Problem p;
  if (!c.cm) {
    p = Problem{c.M, c.N, c.K, c.alpha, c.beta, c.A, c.lda, c.B, c.ldb, c.C, c.ldc, c.sA, c.sB, c.sC, c.ta, c.tb};
  } else {
    p = Problem{c.N, c.M, c.K, c.alpha, c.beta, c.B, c.ldb, c.A, c.lda, c.C, c.ldc, c.sB, c.sA, c.sC, c.tb, c.ta};
  }
  // a workspace too small or not 16-byte aligned (the fix-up reads it as float4) is not used
  const bool ws_ok = c.ws_bytes >= sgemm_impl::kStreamKBytes && reinterpret_cast<uintptr_t>(c.ws) % 16 == 0;
  float* ws = ws_ok ? static_cast<float*>(c.ws) : nullptr;
  if (use_scratch) {
    // the library's static scratch stands in for the caller's workspace, for the calls
    // whose kernels use one (a call that launches nothing, or no stream-K, touches no
    // scratch and makes no lookup)
    const long long need = workspace_need(p, c.batch, c.variant);
    if (need > kScratchBytes) return SGEMM_RM_ERR_SCRATCH_LIMIT;
    if (need > 0) {
      const hipError_t err = scratch_on(stream, &ws);
      if (err != hipSuccess) return (int)err;
    }
  }
  return launch(p, c.batch, stream, c.variant, ws);
}

}  // namespace

// The direct loops (direct_mask) of a query's problem, with its operands as torch allocates
// them: row-major, 16-byte aligned rows.
static int query_direct(int K) {
  return (K % 16 == 0 ? sgemm_impl::kDirect256 | sgemm_impl::kDirect128 : 0) | (K % 32 == 0 ? sgemm_impl::kDirect64 : 0);
}

extern "C" {

int sgemm_rm(int M, int N, int K, float alpha, const float* A, int lda, const float* B, int ldb, float beta,
             float* C, int ldc, hipStream_t stream) {
  return run({false, 0, 0, M, N, K, alpha, A, lda, 0, B, ldb, 0, beta, C, ldc, 0, 1, nullptr, 0,
              SGEMM_RM_VARIANT_AUTO},
             kPosRm, stream);
}

int sgemm_rm_ex(int M, int N, int K, float alpha, const float* A, int lda, const float* B, int ldb, float beta,
                float* C, int ldc, hipStream_t stream, int variant) {
  return run({false, 0, 0, M, N, K, alpha, A, lda, 0, B, ldb, 0, beta, C, ldc, 0, 1, nullptr, 0, variant}, kPosRm,
             stream);
}

int sgemm_rm_strided_batched(int M, int N, int K, float alpha, const float* A, int lda, long long strideA,
                             const float* B, int ldb, long long strideB, float beta, float* C, int ldc,
                             long long strideC, int batch, hipStream_t stream) {
  return run({false, 0, 0, M, N, K, alpha, A, lda, strideA, B, ldb, strideB, beta, C, ldc, strideC, batch,
              nullptr, 0, SGEMM_RM_VARIANT_AUTO},
             kPosRmBatched, stream);
}

int sgemm_rm_strided_batched_ex(int M, int N, int K, float alpha, const float* A, int lda, long long strideA,
                                const float* B, int ldb, long long strideB, float beta, float* C, int ldc,
                                long long strideC, int batch, hipStream_t stream, int variant) {
  return run({false, 0, 0, M, N, K, alpha, A, lda, strideA, B, ldb, strideB, beta, C, ldc, strideC, batch, nullptr,
              0, variant},
             kPosRmBatched, stream);
}

int sgemm_rm_op(int transA, int transB, int M, int N, int K, float alpha, const float* A, int lda, const float* B,
                int ldb, float beta, float* C, int ldc, hipStream_t stream) {
  return run({false, transA, transB, M, N, K, alpha, A, lda, 0, B, ldb, 0, beta, C, ldc, 0, 1, nullptr,
              0, SGEMM_RM_VARIANT_AUTO},
             kPosOp, stream);
}

int sgemm_rm_op_strided_batched_ex(int transA, int transB, int M, int N, int K, float alpha, const float* A,
                                   int lda, long long strideA, const float* B, int ldb, long long strideB,
                                   float beta, float* C, int ldc, long long strideC, int batch, hipStream_t stream,
                                   int variant) {
  return run({false, transA, transB, M, N, K, alpha, A, lda, strideA, B, ldb, strideB, beta, C, ldc, strideC, batch,
              nullptr, 0, variant},
             kPosOpBatched, stream);
}

int sgemm_cm(int transA, int transB, int M, int N, int K, float alpha, const float* A, int lda, const float* B,
             int ldb, float beta, float* C, int ldc, hipStream_t stream) {
  return run({true, transA, transB, M, N, K, alpha, A, lda, 0, B, ldb, 0, beta, C, ldc, 0, 1, nullptr,
              0, SGEMM_RM_VARIANT_AUTO},
             kPosOp, stream);
}

int sgemm_cm_strided_batched_ex(int transA, int transB, int M, int N, int K, float alpha, const float* A, int lda,
                                long long strideA, const float* B, int ldb, long long strideB, float beta, float* C,
                                int ldc, long long strideC, int batch, hipStream_t stream, int variant) {
  return run({true, transA, transB, M, N, K, alpha, A, lda, strideA, B, ldb, strideB, beta, C, ldc, strideC, batch,
              nullptr, 0, variant},
             kPosOpBatched, stream);
}

int sgemm_rm_op_strided_batched_ws(int transA, int transB, int M, int N, int K, float alpha, const float* A,
                                   int lda, long long strideA, const float* B, int ldb, long long strideB,
                                   float beta, float* C, int ldc, long long strideC, int batch, void* workspace,
                                   long long workspace_bytes, hipStream_t stream, int variant) {
  return run({false, transA, transB, M, N, K, alpha, A, lda, strideA, B, ldb, strideB, beta, C, ldc, strideC, batch,
              workspace, workspace_bytes, variant},
             kPosOpBatchedWs, stream);
}

int sgemm_cm_strided_batched_ws(int transA, int transB, int M, int N, int K, float alpha, const float* A, int lda,
                                long long strideA, const float* B, int ldb, long long strideB, float beta, float* C,
                                int ldc, long long strideC, int batch, void* workspace, long long workspace_bytes,
                                hipStream_t stream, int variant) {
  return run({true, transA, transB, M, N, K, alpha, A, lda, strideA, B, ldb, strideB, beta, C, ldc, strideC, batch,
              workspace, workspace_bytes, variant},
             kPosOpBatchedWs, stream);
}

int sgemm_rm_op_strided_batched_noalloc(int transA, int transB, int M, int N, int K, float alpha, const float* A,
                                        int lda, long long strideA, const float* B, int ldb, long long strideB,
                                        float beta, float* C, int ldc, long long strideC, int batch,
                                        hipStream_t stream, int variant) {
  return run({false, transA, transB, M, N, K, alpha, A, lda, strideA, B, ldb, strideB, beta, C, ldc, strideC, batch,
              nullptr, 0, variant},
             kPosOpBatched, stream, true);
}

long long sgemm_rm_workspace_size(int M, int N, int K, int batch) {
  if (M < 0) return -1;
  if (N < 0) return -2;
  if (K < 0) return -3;
  if (batch < 0) return -4;
  if (M == 0 || N == 0 || K == 0 || batch == 0) return 0;
  const sgemm_impl::TilePlan plan = sgemm_impl::plan_tiles(M, N, K, batch, true, query_direct(K));
  return plan.stream_k || plan.slices > 1 ? sgemm_impl::kStreamKBytes : 0;
}

int sgemm_rm_plan_tiles(int M, int N, int K, int batch) {
  if (M < 0) return -1;
  if (N < 0) return -2;
  if (K < 0) return -3;
  if (batch < 0) return -4;
  if (M == 0 || N == 0 || K == 0 || batch == 0) return 0;
  return sgemm_impl::plan_tiles(M, N, K, batch < sgemm_impl::kMaxBatch ? batch : sgemm_impl::kMaxBatch, false,
                                query_direct(K))
      .side;
}

const char* sgemm_rm_strerror(int code) {
  static const char* const kInvalid[] = {
      "invalid argument 1",  "invalid argument 2",  "invalid argument 3",  "invalid argument 4",
      "invalid argument 5",  "invalid argument 6",  "invalid argument 7",  "invalid argument 8",
      "invalid argument 9",  "invalid argument 10", "invalid argument 11", "invalid argument 12",
      "invalid argument 13", "invalid argument 14", "invalid argument 15", "invalid argument 16",
      "invalid argument 17", "invalid argument 18", "invalid argument 19", "invalid argument 20",
      "invalid argument 21"};
  if (code == 0) return "success";
  if (code < 0 && code >= -21) return kInvalid[-code - 1];
  if (code == SGEMM_RM_ERR_SCRATCH_LIMIT) return "the problem needs more scratch than SGEMM_RM_SCRATCH_BYTES";
  if (code > 0) return hipGetErrorString((hipError_t)code);
  return "unknown error code";
}

int sgemm_rm_version(void) { return 400; }

}  // extern "C"
