/*
 * sgemm_rm.h: row-major single-precision GEMM on AMD Instinct MI355X (gfx950).
 *
 *     C := alpha * A * B + beta * C
 *
 * A is M x K, B is K x N and C is M x N, all float32 and row-major with
 * leading dimensions: element (i, j) of X lives at X[i*ldX + j].  This is the
 * operation defined at the top of "Deep dive into the sgemmNN algorithm"
 * (lazypool-blog; C = alpha*A*B + beta*C, A is m x k, B is k x n, C is
 * m x n), with the row-major indexing of the one-thread-per-element kernels
 * in m.lqnn.cn/news/94381 section 1.1 and "GPU-accelerated matrix computation
 * optimisation and CUDA programming practice" section 3.1, and the lda / ldb /
 * ldc arguments of the sgemmNN kernel's signature.
 *
 * Ownership: the caller owns every buffer.  A, B and C are device pointers
 * (hipMalloc'd or equivalent, e.g. a PyTorch tensor's data pointer on the
 * current device).  The library never allocates, frees or retains them and
 * writes only the M x N window of C: columns N..ldc-1 of C are never touched,
 * and A and B are only read within their logical M x K and K x N windows.
 * C must not overlap A or B.
 *
 * Streams: every call only enqueues work on `stream` (0 = the null stream)
 * and returns; the caller synchronises.  Calls are reentrant; the library
 * keeps no state beyond cached device properties.
 *
 * Special cases (BLAS convention; the pages say nothing about them):
 *   - M == 0 or N == 0: nothing is launched.
 *   - alpha == 0 or K == 0: C := beta * C and A, B are not read (they may be
 *     NULL); with beta == 1 nothing is launched.
 *   - beta == 0: C is written without being read, so NaN or Inf in the
 *     initial C does not reach the result.
 *
 * Results match the definition within
 *     |C_gpu(i,j) - C(i,j)| <= 1e-5 * sum_k |A(i,k)| |B(k,j)| + 1e-6;
 * the summation order is fixed per variant and shape, so repeated calls with
 * the same inputs are bitwise identical.
 *
 * Transposed operands and column-major storage (sgemm_rm_op, sgemm_cm and their
 * batched forms) follow the BLAS operation arguments of the cuBLAS calls on
 * "GPU-accelerated matrix computation ..." section 4.1 (CUBLAS_OP_N / _T) and
 * the sgemmNN page, which is the NN member of that column-major family:
 *     C := alpha * op(A) * op(B) + beta * C,   op(X) = X or X^T,
 * op(A) M x K, op(B) K x N, C M x N.  A column-major product is computed as the
 * row-major product C^T = op(B)^T op(A)^T over the same memory.
 *
 * Return value: 0 on success.  A negative value -p names the first invalid
 * argument by its 1-based position p in the call's parameter list, checked in
 * that order before any HIP call.  For sgemm_rm / sgemm_rm_ex:
 *   -1 M < 0          -2 N < 0            -3 K < 0
 *   -5 A == NULL while A is read          -6 lda < max(1, K)
 *   -7 B == NULL while B is read          -8 ldb < max(1, N)
 *   -10 C == NULL while M*N > 0           -11 ldc < max(1, N)
 *   -13 (sgemm_rm_ex only) unknown variant
 * For the strided-batched calls see their declarations.  A positive value is
 * the hipError_t reported by the HIP runtime for a launch (the analogue of
 * checking cudaGetLastError after a launch, which the mlqm.cn/news/1180856
 * troubleshooting table, section 7, recommends).
 */
#ifndef SGEMM_RM_H
#define SGEMM_RM_H

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Kernel families, in the order the pages build them up. */
enum sgemm_rm_variant {
  SGEMM_RM_VARIANT_AUTO = 0,      /* library's choice for the shape (MFMA + edge path) */
  SGEMM_RM_VARIANT_NAIVE = 1,     /* one thread per C element, m.lqnn.cn/news/94381 section 1.1 */
  SGEMM_RM_VARIANT_LDS_TILED = 2, /* LDS tiles, 128-bit loads, zero-filled edges, padded rows:
                                     m.lqnn.cn/news/94381 sections 2-5 */
  SGEMM_RM_VARIANT_REGBLOCK = 3,  /* register-blocked, double-buffered LDS pipeline:
                                     "GEMM advanced: ILP and bank conflicts" (mhpn.cn) section 2-3,
                                     and the sgemmNN page's register blocking */
  SGEMM_RM_VARIANT_MFMA = 4,      /* FP32 matrix-core tiles for full tiles, scalar edge-tile path
                                     for ragged M/N; ragged K handled inside every tile; tile
                                     configuration chosen per shape (sgemm_rm_plan_tiles) */
  /* The MFMA kernel with its tile configuration forced, for tile sweeps (the pages name
     tuning the tile parameters as the next step: the sgemmNN page's closing section): */
  SGEMM_RM_VARIANT_MFMA_T256 = 5, /* 256 x 256 tiles, one workgroup per CU (8 or 4 wavefronts) */
  SGEMM_RM_VARIANT_MFMA_T128 = 6, /* 128 x 128 tiles, two workgroups of 4 wavefronts per CU (8 at one tile per CU) */
  SGEMM_RM_VARIANT_MFMA_T64 = 7,  /* 64 x 64 tiles, 4 x 32 x 32 wavefronts, 2-way in-tile K split */
  SGEMM_RM_VARIANT_MFMA_T32 = 8,  /* 32 x 32 tiles, 4-way in-tile K split */
  SGEMM_RM_VARIANT_MFMA_T192 = 9, /* 192 x 192 tiles, 4 wavefronts of 96 x 96, one workgroup per CU */
  SGEMM_RM_VARIANT_MFMA_T16 = 10  /* 16 x 16 blocks on 16x16x4 MFMA, K split over 8 wavefronts */
};

/*
 * C := alpha*A*B + beta*C (row-major, leading dimensions), asynchronously on
 * `stream`, with the library's choice of kernels for the shape.
 */
int sgemm_rm(int M, int N, int K, float alpha, const float* A, int lda, const float* B, int ldb,
             float beta, float* C, int ldc, hipStream_t stream);

/*
 * As sgemm_rm, with the kernel family forced (enum sgemm_rm_variant).  Every
 * variant accepts every valid shape, leading dimension and 4-byte-aligned
 * pointer; 128-bit global loads are used only where the base pointers, the
 * leading dimensions and, in the batched calls, the batch strides keep them
 * 16-byte aligned.  Every call is one or a few launches on `stream`: a C window
 * whose tiled launch could need 2^32 or more work-items (M rounded up to 16 times
 * ceil(N / 16) above 2^27 - 1: about 2^31 elements, fewer for windows narrower
 * than 16 columns) runs, in the tiled families, as bands of rows (and of columns
 * for rows of more than about 2.8 million elements) launched one after another,
 * band edges on multiples of 768 rows and columns, so that no grid exceeds the
 * 32-bit work-item count of a dispatch; the naive family and the C := beta*C pass
 * of alpha == 0 or K == 0 take any window in one launch.
 */
int sgemm_rm_ex(int M, int N, int K, float alpha, const float* A, int lda, const float* B, int ldb,
                float beta, float* C, int ldc, hipStream_t stream, int variant);

/*
 * Strided batch of independent GEMMs, all with the same M, N, K, alpha, beta and
 * leading dimensions (the strided-batched form of "GPU-accelerated matrix
 * computation ..." section 4.2, which batches many small products in one call):
 *
 *     for b in [0, batch):  C_b := alpha * A_b * B_b + beta * C_b
 *     A_b = A + b*strideA,  B_b = B + b*strideB,  C_b = C + b*strideC   (in floats)
 *
 * Strides may be 0 for A or B (the same operand for every entry).  The C
 * matrices of different entries must not overlap: strideC >= (M-1)*ldc + N
 * when batch > 1.  One launch covers up to 65535 entries; larger batches are
 * split into several launches on the same stream.  Return codes, by position:
 *   -1 M, -2 N, -3 K < 0; -5 A NULL while read; -6 lda < max(1,K);
 *   -7 strideA < 0; -8 B NULL while read; -9 ldb < max(1,N); -10 strideB < 0;
 *   -12 C NULL while written; -13 ldc < max(1,N); -14 strideC < 0 or outputs
 *   overlap; -15 batch < 0; -17 (the _ex form) unknown variant.
 */
int sgemm_rm_strided_batched(int M, int N, int K, float alpha, const float* A, int lda, long long strideA,
                             const float* B, int ldb, long long strideB, float beta, float* C, int ldc,
                             long long strideC, int batch, hipStream_t stream);

/* As sgemm_rm_strided_batched, with the kernel family forced (enum sgemm_rm_variant). */
int sgemm_rm_strided_batched_ex(int M, int N, int K, float alpha, const float* A, int lda, long long strideA,
                                const float* B, int ldb, long long strideB, float beta, float* C, int ldc,
                                long long strideC, int batch, hipStream_t stream, int variant);

/* Operation arguments of the transposing calls. */
enum sgemm_rm_op {
  SGEMM_RM_OP_N = 0, /* op(X) = X */
  SGEMM_RM_OP_T = 1  /* op(X) = X^T */
};

/*
 * C := alpha * op(A) * op(B) + beta * C, all row-major (element (i, j) of X at
 * X[i*ldX + j]).  transA == SGEMM_RM_OP_N: A is stored M x K, lda >= max(1, K);
 * SGEMM_RM_OP_T: A is stored K x M (op(A)(i, k) = A[k*lda + i]), lda >= max(1, M).
 * transB == SGEMM_RM_OP_N: B stored K x N, ldb >= max(1, N); SGEMM_RM_OP_T: B
 * stored N x K, ldb >= max(1, K).  C is M x N, ldc >= max(1, N).  Every kernel
 * family reads transposed operands along their contiguous dimension; the
 * MFMA kernel keeps each operand's LDS layout matched to its storage order.
 * Return codes, by position: -1 transA, -2 transB not 0 or 1; -3 M, -4 N,
 * -5 K < 0; -7 A NULL while read; -8 lda too small; -9 B NULL while read;
 * -10 ldb too small; -12 C NULL while written; -13 ldc < max(1, N).
 * With both flags SGEMM_RM_OP_N this is sgemm_rm.
 */
int sgemm_rm_op(int transA, int transB, int M, int N, int K, float alpha, const float* A, int lda, const float* B,
                int ldb, float beta, float* C, int ldc, hipStream_t stream);

/*
 * The general row-major call: a strided batch (as sgemm_rm_strided_batched) of
 * C_b := alpha * op(A_b) * op(B_b) + beta * C_b with the operation arguments and
 * leading-dimension rules of sgemm_rm_op and the kernel family forced (enum
 * sgemm_rm_variant).  Return codes, by position: -1 transA, -2 transB; -3 M,
 * -4 N, -5 K < 0; -7 A NULL while read; -8 lda too small; -9 strideA < 0;
 * -10 B NULL while read; -11 ldb too small; -12 strideB < 0; -14 C NULL while
 * written; -15 ldc < max(1, N); -16 strideC < 0 or outputs overlap
 * (strideC < (M-1)*ldc + N with batch > 1); -17 batch < 0; -19 unknown variant.
 */
int sgemm_rm_op_strided_batched_ex(int transA, int transB, int M, int N, int K, float alpha, const float* A,
                                   int lda, long long strideA, const float* B, int ldb, long long strideB,
                                   float beta, float* C, int ldc, long long strideC, int batch, hipStream_t stream,
                                   int variant);

/*
 * Column-major (BLAS) form: C := alpha * op(A) * op(B) + beta * C with element
 * (i, j) of X at X[j*ldX + i].  transA == SGEMM_RM_OP_N: A is M x K, lda >=
 * max(1, M); SGEMM_RM_OP_T: A is stored K x M, lda >= max(1, K).  transB ==
 * SGEMM_RM_OP_N: B is K x N, ldb >= max(1, K); SGEMM_RM_OP_T: B is stored N x K,
 * ldb >= max(1, N).  C is M x N, ldc >= max(1, M).  Same argument order and
 * return codes as sgemm_rm_op (-13: ldc < max(1, M)).  The sgemmNN page's
 * kernel computes the (N, N) case of this call.
 */
int sgemm_cm(int transA, int transB, int M, int N, int K, float alpha, const float* A, int lda, const float* B,
             int ldb, float beta, float* C, int ldc, hipStream_t stream);

/*
 * Strided batch of sgemm_cm problems with the kernel family forced; argument
 * order and return codes as sgemm_rm_op_strided_batched_ex, except that the
 * outputs overlap (-16) when batch > 1 and strideC < (N-1)*ldc + M.
 */
int sgemm_cm_strided_batched_ex(int transA, int transB, int M, int N, int K, float alpha, const float* A, int lda,
                                long long strideA, const float* B, int ldb, long long strideB, float beta, float* C,
                                int ldc, long long strideC, int batch, hipStream_t stream, int variant);

/*
 * The general row-major call with a caller-owned workspace: as
 * sgemm_rm_op_strided_batched_ex, and, for a single product, where the library's cost
 * model expects it to be faster: (a) where its 256 x 256 tiles leave the last wave of 256
 * workgroups partly empty, the last waves run as "stream-K" (their K-tiles shared evenly
 * by 256 workgroups; after the Stream-K work decomposition, not a technique of the
 * pages); (b) where a product of few 64 x 64 tiles has a long K (e.g. 256 x 256 x 65536),
 * each tile's K range is cut into slices, one workgroup each, so that the CUs fill ("K
 * slices", the deterministic split-K that small outputs call for).  Partial tiles go to
 * `workspace` (device memory, at least sgemm_rm_workspace_size bytes; the library only
 * writes and reads it during the call's kernels) and a second kernel adds them in a fixed
 * order, so results are deterministic; their summation order, and so their rounding,
 * differs from the call without a workspace.  With workspace NULL, not 16-byte aligned
 * (hipMalloc gives 256) or workspace_bytes below the size needed, the call is exactly
 * sgemm_rm_op_strided_batched_ex.  With a large enough workspace, SGEMM_RM_VARIANT_MFMA_T256
 * uses stream-K whenever the tiles leave a partial wave and SGEMM_RM_VARIANT_MFMA_T64 uses
 * K slices wherever they apply (a single product covered by 64 x 64 tiles, remainders of
 * 0 or at least 16 rows and columns, whose tiles fill under one workgroup per CU and whose
 * K gives each slice at least 512), for tests and sweeps; the other forced variants ignore
 * the workspace.  Calls that share a
 * workspace must not overlap (same stream, or synchronised).  Return codes as
 * sgemm_rm_op_strided_batched_ex, plus -18 workspace NULL with workspace_bytes > 0,
 * -19 workspace_bytes < 0; the stream is argument 20 and -21 is an unknown variant.
 */
int sgemm_rm_op_strided_batched_ws(int transA, int transB, int M, int N, int K, float alpha, const float* A,
                                   int lda, long long strideA, const float* B, int ldb, long long strideB,
                                   float beta, float* C, int ldc, long long strideC, int batch, void* workspace,
                                   long long workspace_bytes, hipStream_t stream, int variant);

/* The column-major form of sgemm_rm_op_strided_batched_ws (rules of sgemm_cm). */
int sgemm_cm_strided_batched_ws(int transA, int transB, int M, int N, int K, float alpha, const float* A, int lda,
                                long long strideA, const float* B, int ldb, long long strideB, float beta, float* C,
                                int ldc, long long strideC, int batch, void* workspace, long long workspace_bytes,
                                hipStream_t stream, int variant);

/*
 * Size of the library's static device scratch (128 MiB per GPU), and the return code of a
 * call that would need more scratch than that.
 */
#define SGEMM_RM_SCRATCH_BYTES (128LL << 20)
#define SGEMM_RM_ERR_SCRATCH_LIMIT (-100)

/*
 * For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): sgemm_rm_op_strided_batched_ws with
 * the library's own static scratch as the workspace.  Same arguments, rules and return
 * codes as sgemm_rm_op_strided_batched_ex (the stream is argument 18, -19 an unknown
 * variant); the kernels, and so the results, are those of sgemm_rm_op_strided_batched_ws
 * given a workspace of SGEMM_RM_SCRATCH_BYTES (stream-K where that call would run it).
 * The call allocates nothing: the scratch is a static __device__ array of
 * SGEMM_RM_SCRATCH_BYTES that each GPU the library runs on holds from the first call
 * until the process ends; its address on a device is looked up (hipGetSymbolAddress)
 * on the first call for that device, with that device made current for the lookup.
 * A problem whose kernels would need more than SGEMM_RM_SCRATCH_BYTES returns
 * SGEMM_RM_ERR_SCRATCH_LIMIT before any launch (every current kernel needs at most
 * that much).  Every call on one GPU shares that GPU's scratch, which keeps the last
 * call's contents; nothing in it has to start at zero.  Calls that may overlap on one
 * GPU (different streams not synchronised, or several host threads) race on the
 * scratch and must be serialised by the caller.  A positive value is a hipError_t
 * (of the lookup or a launch).
 */
int sgemm_rm_op_strided_batched_noalloc(int transA, int transB, int M, int N, int K, float alpha, const float* A,
                                        int lda, long long strideA, const float* B, int ldb, long long strideB,
                                        float beta, float* C, int ldc, long long strideC, int batch,
                                        hipStream_t stream, int variant);

/*
 * Workspace bytes with which the _ws calls run an M x N x K problem (repeated `batch`
 * times) as stream-K or with K slices, or 0 where the cost model keeps the
 * one-tile-per-workgroup path, for operands whose rows are 16-byte aligned (as
 * sgemm_rm_plan_tiles).  Currently 0 or 128 MiB (two 256 x 256 float partial tiles for
 * each of 256 workgroups).  -1 M < 0, -2 N < 0, -3 K < 0, -4 batch < 0.  Host only: no
 * HIP call.  The transpose flags and storage order do not change the answer.
 */
long long sgemm_rm_workspace_size(int M, int N, int K, int batch);

/*
 * Tile side (256, 192, 128, 64, 32 or 16) of the MFMA configuration that SGEMM_RM_VARIANT_AUTO
 * and SGEMM_RM_VARIANT_MFMA use for an M x N x K problem repeated `batch` times (any
 * orientation or storage order; batches above 65535 are planned per launch of 65535), for
 * operands whose rows are 16-byte aligned (pointers and leading dimensions; the 256
 * configuration's partial tiles need such rows, and without them the choice may differ).
 * 0 when nothing would be launched for the product (M, N, K or batch 0).  -1 M < 0,
 * -2 N < 0, -3 K < 0, -4 batch < 0.  Host only: no HIP call.
 */
int sgemm_rm_plan_tiles(int M, int N, int K, int batch);

/* Static, NUL-terminated description of a return code of the calls above
 * ("invalid argument p" for -p, the HIP runtime's text for a hipError_t). */
const char* sgemm_rm_strerror(int code);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int sgemm_rm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SGEMM_RM_H */
