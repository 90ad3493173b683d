/*
 * A plain C client of libsgemm_rm: device buffers from the HIP runtime (no PyTorch),
 * one call through the C ABI, the result written to a file for the test to compare
 * with the oracle.
 *
 *   sgemm_client M N K lda ldb ldc alpha beta variant out.bin
 *
 * Inputs are integers in [-4, 4] from fixed formulas (the test rebuilds them):
 *   A(i, k) = (7i + 3k) mod 9 - 4,  B(k, j) = (5k + 2j + 1) mod 9 - 4,
 *   C(i, j) = (i + 4j + 2) mod 9 - 4; padding columns hold -7.
 * out.bin holds the M x ldc buffer of C after the call (float32, row-major).
 * Before the product the client checks that an invalid lda is rejected with -6
 * before any HIP call.  Exit status 0 on success.
 */
#include <stdio.h>
#include <stdlib.h>

#include <hip/hip_runtime_api.h>

#include "sgemm_rm.h"

static float* fill(int rows, int cols, int ld, int kind) {
  float* h = (float*)malloc(sizeof(float) * (size_t)rows * (size_t)ld);
  if (h == NULL) return NULL;
  for (int r = 0; r < rows; ++r)
    for (int c = 0; c < ld; ++c) {
      int v;
      if (c >= cols) v = -7;
      else if (kind == 0) v = (7 * r + 3 * c) % 9 - 4;
      else if (kind == 1) v = (5 * r + 2 * c + 1) % 9 - 4;
      else v = (r + 4 * c + 2) % 9 - 4;
      h[(size_t)r * ld + c] = (float)v;
    }
  return h;
}

int main(int argc, char** argv) {
  if (argc != 11) {
    fprintf(stderr, "usage: %s M N K lda ldb ldc alpha beta variant out.bin\n", argv[0]);
    return 2;
  }
  const int M = atoi(argv[1]), N = atoi(argv[2]), K = atoi(argv[3]);
  const int lda = atoi(argv[4]), ldb = atoi(argv[5]), ldc = atoi(argv[6]);
  const float alpha = (float)atof(argv[7]), beta = (float)atof(argv[8]);
  const int variant = atoi(argv[9]);

  const int bad = sgemm_rm(M, N, K, alpha, (const float*)16, K > 1 ? K - 1 : 0, (const float*)16, ldb, beta,
                           (float*)16, ldc, NULL);
  if (bad != -6) {
    fprintf(stderr, "invalid lda gave %d (%s), expected -6\n", bad, sgemm_rm_strerror(bad));
    return 3;
  }

  float *hA = fill(M, K, lda, 0), *hB = fill(K, N, ldb, 1), *hC = fill(M, N, ldc, 2);
  if (hA == NULL || hB == NULL || hC == NULL) return 4;
  const size_t sa = sizeof(float) * (size_t)M * lda, sb = sizeof(float) * (size_t)K * ldb,
               sc = sizeof(float) * (size_t)M * ldc;
  float *dA = NULL, *dB = NULL, *dC = NULL;
  if (hipMalloc((void**)&dA, sa) != hipSuccess || hipMalloc((void**)&dB, sb) != hipSuccess ||
      hipMalloc((void**)&dC, sc) != hipSuccess) {
    fprintf(stderr, "hipMalloc failed\n");
    return 5;
  }
  if (hipMemcpy(dA, hA, sa, hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpy(dB, hB, sb, hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpy(dC, hC, sc, hipMemcpyHostToDevice) != hipSuccess)
    return 6;
  hipStream_t stream;
  if (hipStreamCreate(&stream) != hipSuccess) return 7;
  const int rc = sgemm_rm_ex(M, N, K, alpha, dA, lda, dB, ldb, beta, dC, ldc, stream, variant);
  if (rc != 0) {
    fprintf(stderr, "sgemm_rm_ex: %d (%s)\n", rc, sgemm_rm_strerror(rc));
    return 8;
  }
  if (hipStreamSynchronize(stream) != hipSuccess) return 9;
  if (hipMemcpy(hC, dC, sc, hipMemcpyDeviceToHost) != hipSuccess) return 10;
  FILE* f = fopen(argv[10], "wb");
  if (f == NULL || fwrite(hC, 1, sc, f) != sc) return 11;
  fclose(f);
  hipStreamDestroy(stream);
  hipFree(dA);
  hipFree(dB);
  hipFree(dC);
  free(hA);
  free(hB);
  free(hC);
  printf("sgemm_client %dx%dx%d variant %d: ok (library version %d)\n", M, N, K, variant, sgemm_rm_version());
  return 0;
}
