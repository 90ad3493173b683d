// Test aid: records the lane layout of the FP32 MFMA instructions the SGEMM
// kernels use (v_mfma_f32_32x32x2_f32, v_mfma_f32_16x16x4_f32) with one-hot
// operands, so that a test can compare it with the layout the kernels assume.
//
// Launch: 128 workgroups of one 64-lane wavefront.  Workgroup L < 64 sets
// A-operand lane L to 1 (all other A lanes 0) and B-operand lane l to l + 1;
// workgroup 64 + L does the converse.  Each lane stores its 16 (32x32x2) and 4
// (16x16x4) accumulator registers.  Output (binary, float32): the 128*64*16
// values of the 32x32x2 runs, then the 128*64*4 values of the 16x16x4 runs.
//
// Usage: mfma_layout_probe OUTPUT_FILE
#include <hip/hip_runtime.h>

#include <cstdio>
#include <vector>

typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kBlocks = 128;

__global__ __launch_bounds__(64) void probe(float* out32, float* out16) {
  const int L = blockIdx.x & 63;
  const bool onehot_a = blockIdx.x < 64;
  const int l = threadIdx.x;
  const float a = onehot_a ? (l == L ? 1.f : 0.f) : float(l + 1);
  const float b = onehot_a ? float(l + 1) : (l == L ? 1.f : 0.f);
  v16f c = {0};
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  v4f d = {0};
  d = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, d, 0, 0, 0);
  for (int r = 0; r < 16; ++r) out32[(blockIdx.x * 64 + l) * 16 + r] = c[r];
  for (int r = 0; r < 4; ++r) out16[(blockIdx.x * 64 + l) * 4 + r] = d[r];
}

int main(int argc, char** argv) {
  if (argc < 2) {
    fprintf(stderr, "usage: %s OUTPUT_FILE\n", argv[0]);
    return 2;
  }
  std::vector<float> h32(kBlocks * 64 * 16), h16(kBlocks * 64 * 4);
  float *d32 = nullptr, *d16 = nullptr;
  if (hipMalloc(&d32, h32.size() * 4) != hipSuccess || hipMalloc(&d16, h16.size() * 4) != hipSuccess) {
    fprintf(stderr, "hipMalloc failed\n");
    return 1;
  }
  hipLaunchKernelGGL(probe, dim3(kBlocks), dim3(64), 0, 0, d32, d16);
  if (hipDeviceSynchronize() != hipSuccess ||
      hipMemcpy(h32.data(), d32, h32.size() * 4, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(h16.data(), d16, h16.size() * 4, hipMemcpyDeviceToHost) != hipSuccess) {
    fprintf(stderr, "probe failed\n");
    return 1;
  }
  FILE* f = fopen(argv[1], "wb");
  if (!f) return 1;
  fwrite(h32.data(), 4, h32.size(), f);
  fwrite(h16.data(), 4, h16.size(), f);
  fclose(f);
  printf("wrote %zu floats\n", h32.size() + h16.size());
  return (hipFree(d32) == hipSuccess && hipFree(d16) == hipSuccess) ? 0 : 1;
}
