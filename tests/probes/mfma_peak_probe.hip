// Test aid: the FP32 matrix-core throughput a kernel can reach with no memory traffic.
//
// Every wavefront runs ITERS rounds of CHAINS independent v_mfma_f32_32x32x2_f32
// (4096 FLOP each) on register operands; 256 workgroups x WAVES wavefronts.  The
// printed TFLOP/s is the ceiling the SGEMM kernels' own MFMA sequences run under
// (issue and dependency limits included), to set beside 157.3 TFLOP/s.
//
// Usage: mfma_peak_probe  (prints "chains=C waves_per_simd=W tflops=T" lines)
#include <hip/hip_runtime.h>

#include <cstdio>

typedef float v16f __attribute__((ext_vector_type(16)));

template <int CHAINS>
__global__ __launch_bounds__(1024) void peak(int iters, float* sink) {
  v16f acc[CHAINS];
#pragma unroll
  for (int c = 0; c < CHAINS; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
  float a = 1.0f + threadIdx.x * 1e-7f, b = 0.5f - threadIdx.x * 1e-7f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < CHAINS; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < CHAINS; ++c) s += acc[c][0];
  if (s == -1.f) sink[threadIdx.x] = s;
}

template <int CHAINS>
static int run(int waves_per_simd, float* sink, double clock_hz, int cus) {
  const int threads = waves_per_simd * 4 * 64, blocks = cus, iters = 20000 / CHAINS;
  hipEvent_t a, b;
  if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) return 1;
  for (int rep = 0; rep < 3; ++rep) {
    if (hipEventRecord(a) != hipSuccess) return 1;
    hipLaunchKernelGGL(peak<CHAINS>, dim3(blocks), dim3(threads), 0, 0, iters, sink);
    if (hipEventRecord(b) != hipSuccess || hipEventSynchronize(b) != hipSuccess) return 1;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, a, b) != hipSuccess) return 1;
    const double flop = 4096.0 * CHAINS * iters * (threads / 64) * blocks;
    if (rep == 2)
      printf("chains=%d waves_per_simd=%d ms=%.3f tflops=%.2f (peak at %.2f GHz: %.2f)\n", CHAINS, waves_per_simd, ms,
             flop / (ms * 1e-3) / 1e12, clock_hz / 1e9, cus * 4 * 64.0 * clock_hz / 1e12);
  }
  return 0;
}

int main() {
  float* sink = nullptr;
  if (hipMalloc(&sink, 1024 * sizeof(float)) != hipSuccess) return 1;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, 0) != hipSuccess) return 1;
  const double clk = prop.clockRate * 1e3;
  const int cus = prop.multiProcessorCount;
  int rc = 0;
  for (int w : {1, 2, 4}) {
    rc |= run<1>(w, sink, clk, cus);
    rc |= run<2>(w, sink, clk, cus);
    rc |= run<4>(w, sink, clk, cus);
    rc |= run<8>(w, sink, clk, cus);
  }
  return rc | (hipFree(sink) != hipSuccess);
}
