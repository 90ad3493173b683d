// Test aid: what the MFMA schedule of a K-tile costs, with no global memory.
//
// 256 workgroups of WAVES wavefronts run `tiles` rounds of the K-tile body of the MFMA
// SGEMM kernel: each wavefront owns FM x FN accumulator blocks of 32 x 32 and issues
// 8 * FM * FN v_mfma_f32_32x32x2_f32 per round (every configuration below gives each SIMD
// 128 MFMAs per round).  Optionally each round ends with a workgroup barrier (BARRIER) and
// reads its MFMA fragments from LDS right before the MFMAs (LDSREAD: two 128-bit A reads
// and eight 32-bit B reads per 32 x 32 block and lane, the kernel's layout), so the cost of
// each part of the schedule shows against the bare MFMA rate.
//
// Usage: mfma_schedule_probe  (prints one line per configuration, ending in TFLOP/s)
#include <hip/hip_runtime.h>
#include <cstdio>
typedef float v16f __attribute__((ext_vector_type(16)));

template <int FM, int FN, int WAVES, bool BARRIER, bool LDSREAD>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(WAVES / 4)))
void probe(int tiles, float* sink) {
  constexpr int ROWS = 64 * 4;  // a 256-row fragment area, 16 floats per row (A-like), and a B-like area
  __shared__ __attribute__((aligned(16))) float lds[2][ROWS * 16 + 16 * (ROWS + 4)];
  for (int i = threadIdx.x; i < 2 * (ROWS * 16 + 16 * (ROWS + 4)); i += WAVES * 64)
    (&lds[0][0])[i] = 1e-3f * (i % 97);
  __syncthreads();
  const int l = threadIdx.x % 64, w = threadIdx.x / 64;
  const int lr = l % 32, lh = l / 32;
  v16f acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  float af[FM][8], bf[FN][8];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) af[i][e] = 1.0f + 1e-7f * (threadIdx.x + i + e);
#pragma unroll
  for (int j = 0; j < FN; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) bf[j][e] = 0.5f - 1e-7f * (threadIdx.x + j + e);
  const int wm0 = (w % 4) * 32 * FM % ROWS, wn0 = (w / 4) * 32 * FN % ROWS;
  for (int t = 0; t < tiles; ++t) {
    if (LDSREAD) {
      const float* A = lds[t & 1];
      const float* B = lds[t & 1] + ROWS * 16;
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int rr = (wm0 + i * 32 + lr) % ROWS;
        const float4 x0 = *reinterpret_cast<const float4*>(A + rr * 16 + 4 * ((2 * lh) ^ ((rr / 4) & 3)));
        const float4 x1 = *reinterpret_cast<const float4*>(A + rr * 16 + 4 * ((2 * lh + 1) ^ ((rr / 4) & 3)));
        af[i][0] = x0.x; af[i][1] = x0.y; af[i][2] = x0.z; af[i][3] = x0.w;
        af[i][4] = x1.x; af[i][5] = x1.y; af[i][6] = x1.z; af[i][7] = x1.w;
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int cc = (wn0 + j * 32 + lr) % ROWS;
#pragma unroll
        for (int e = 0; e < 8; ++e) bf[j][e] = B[(8 * lh + e) * (ROWS + 4) + cc];
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[i][e], bf[j][e], acc[i][j], 0, 0, 0);
    if (BARRIER) __syncthreads();
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) s += acc[i][j][0] + acc[i][j][15];
  if (s == -1.f) sink[threadIdx.x] = s;
}

template <int FM, int FN, int WAVES, bool BARRIER, bool LDSREAD>
static int run(float* sink, int cus, const char* name) {
  const int tiles = 4096;
  hipEvent_t a, b;
  if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) return 1;
  float best = 1e30f;
  for (int rep = 0; rep < 4; ++rep) {
    if (hipEventRecord(a) != hipSuccess) return 1;
    hipLaunchKernelGGL((probe<FM, FN, WAVES, BARRIER, LDSREAD>), dim3(cus), dim3(WAVES * 64), 0, 0, tiles, sink);
    if (hipGetLastError() != hipSuccess) return 1;
    if (hipEventRecord(b) != hipSuccess || hipEventSynchronize(b) != hipSuccess) return 1;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, a, b) != hipSuccess) return 1;
    if (rep > 0 && ms < best) best = ms;
  }
  const double flop = 4096.0 * 8 * FM * FN * (double)WAVES * tiles * cus;
  printf("%-40s waves/SIMD=%d acc_blocks=%2d barrier=%d lds=%d  %.3f ms  %.2f TFLOP/s\n", name, WAVES / 4, FM * FN,
         (int)BARRIER, (int)LDSREAD, best, flop / (best * 1e-3) / 1e12);
  return 0;
}

#define RUN4(FM, FN, W, NAME)                          \
  rc |= run<FM, FN, W, false, false>(sink, cus, NAME); \
  rc |= run<FM, FN, W, true, false>(sink, cus, NAME);  \
  rc |= run<FM, FN, W, false, true>(sink, cus, NAME);  \
  rc |= run<FM, FN, W, true, true>(sink, cus, NAME);

int main() {
  float* sink = nullptr;
  if (hipMalloc(&sink, 4096 * sizeof(float)) != hipSuccess) return 1;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, 0) != hipSuccess) return 1;
  const int cus = prop.multiProcessorCount;
  int rc = 0;
  RUN4(2, 2, 16, "64x64/wave, 16 waves")
  RUN4(4, 2, 8, "128x64/wave, 8 waves")
  RUN4(4, 4, 4, "128x128/wave, 4 waves")
  RUN4(2, 2, 4, "64x64/wave, 4 waves")
  RUN4(4, 2, 4, "128x64/wave, 4 waves")
  return rc | (hipFree(sink) != hipSuccess);
}
