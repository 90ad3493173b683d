// Test aid: LDS bank behaviour of gfx950 for 32-, 64- and 128-bit reads.
//
// Every lane l of every wavefront repeatedly reads LDS word (l * s * W) mod
// 16384 (W = 1, 2, 4 words per access) for a lane stride s; the kernel time
// gives the CU cycles one wavefront-wide read costs.  A conflict-free pattern
// costs the minimum for its width; a pattern whose lanes share banks costs
// proportionally more.  The same binary under rocprofv3 --pmc
// SQ_LDS_BANK_CONFLICT is the positive control for that counter.
//
// Launch: 2048 workgroups of 256 threads, 64 KiB of LDS each; every address
// is (l*s*W) & (16384 - W) words, inside the array and W-aligned.
// Usage: lds_bank_probe  (prints "width=W stride=s cycles=c" lines)
#include <hip/hip_runtime.h>

#include <cstdio>

template <int W>
struct VT;
template <>
struct VT<1> {
  typedef float T;
};
template <>
struct VT<2> {
  typedef float2 T;
};
template <>
struct VT<4> {
  typedef float4 T;
};

constexpr int kWords = 16384;

template <int W>
__global__ __launch_bounds__(256) void probe(int stride, int iters, float* sink) {
  __shared__ __attribute__((aligned(16))) float lds[kWords];
  for (int i = threadIdx.x; i < kWords; i += 256) lds[i] = (float)i;
  __syncthreads();
  const int l = threadIdx.x % 64;
  const int addr = (l * stride * W) & (kWords - W);
  typedef typename VT<W>::T T;
  const T* v = reinterpret_cast<const T*>(lds + addr);
  float acc = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const T x = *v;
      asm volatile("" ::: "memory");  // keep every read
      if constexpr (W == 1)
        acc += x;
      else if constexpr (W == 2)
        acc += x.x + x.y;
      else
        acc += x.x + x.y + x.z + x.w;
    }
  }
  if (acc == -1.f) sink[threadIdx.x] = acc;
}

int main() {
  float* sink = nullptr;
  if (hipMalloc(&sink, 256 * sizeof(float)) != hipSuccess) return 1;
  hipEvent_t a, b;
  if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) return 1;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, 0) != hipSuccess) return 1;
  const int iters = 2000, blocks = 2048;
  const int strides[] = {0, 1, 2, 3, 4, 5, 8, 9, 16, 17, 32, 33, 64, 65};
  for (int w : {1, 2, 4}) {
    for (int s : strides) {
      float ms = 0.f;
      for (int rep = 0; rep < 2; ++rep) {  // second run is timed
        if (hipEventRecord(a) != hipSuccess) return 1;
        if (w == 1) hipLaunchKernelGGL(probe<1>, dim3(blocks), dim3(256), 0, 0, s, iters, sink);
        if (w == 2) hipLaunchKernelGGL(probe<2>, dim3(blocks), dim3(256), 0, 0, s, iters, sink);
        if (w == 4) hipLaunchKernelGGL(probe<4>, dim3(blocks), dim3(256), 0, 0, s, iters, sink);
        if (hipEventRecord(b) != hipSuccess || hipEventSynchronize(b) != hipSuccess) return 1;
        if (hipEventElapsedTime(&ms, a, b) != hipSuccess) return 1;
      }
      const double wave_reads = (double)blocks * 4 * iters * 8;
      const double cycles = ms * 1e-3 * (prop.clockRate * 1e3) * prop.multiProcessorCount / wave_reads;
      printf("width=%d stride=%d ms=%.3f cycles=%.2f\n", w, s, ms, cycles);
    }
  }
  return hipFree(sink) == hipSuccess ? 0 : 1;
}
