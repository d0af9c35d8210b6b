// MFMA-rate reference for the MFMA-bound kernels' rooflines: how many fp16
// flops per second the matrix cores of this GPU sustain on a kernel that does
// nothing but v_mfma_f32_32x32x16_f16, and at what shader clock.
//
// Each wave runs `iters` rounds of 8 independent MFMAs (8 accumulator chains,
// so no product waits for the previous one's result) on operands held in
// registers; the launch has 2 workgroups of 4 waves per CU, as the decode
// attention kernel does. Every wave reads the shader cycle counter and the
// constant-rate counter at its start and end, so the clock the MFMAs ran at
// comes with the rate. The accumulators are folded into one value that is
// written only if it equals a constant they never produce, so the products
// cannot be dropped.
//
// Usage: mfma_rate [iters]   (default 20000)
// One JSON line: mean time of a launch (back to back, after one warm-up),
// the fp16 TFLOP/s it sustains, the mean shader clock over the waves.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>

#define CK(x)                                                                       \
  do {                                                                              \
    hipError_t e_ = (x);                                                            \
    if (e_ != hipSuccess) {                                                         \
      fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      return 1;                                                                     \
    }                                                                               \
  } while (0)

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float16v __attribute__((ext_vector_type(16)));
constexpr int kChains = 8;

__global__ __launch_bounds__(256, 2) void mfma_kernel(int iters, float* out, unsigned long long* ticks) {
  const int l = threadIdx.x & 63;
  half8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (_Float16)(0.001f * (l + i));
    b[i] = (_Float16)(0.002f * (l - i));
  }
  float16v acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = float16v{};
  const unsigned long long c0 = clock64(), r0 = wall_clock64();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[c], 0, 0, 0);
  }
  const unsigned long long c1 = clock64(), r1 = wall_clock64();
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[c][i];
  if (s == 1234.5678f) out[blockIdx.x * blockDim.x + threadIdx.x] = s;
  if (l == 0) {
    const int w = blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
    ticks[2 * w] = c1 - c0;
    ticks[2 * w + 1] = r1 - r0;
  }
}

int main(int argc, char** argv) {
  const int iters = argc > 1 ? atoi(argv[1]) : 20000;
  if (iters < 1 || iters > 10000000) {
    fprintf(stderr, "iters out of range\n");
    return 2;
  }
  int dev = 0, n_cu = 0, wall_khz = 0;
  CK(hipGetDevice(&dev));
  CK(hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev));
  CK(hipDeviceGetAttribute(&wall_khz, hipDeviceAttributeWallClockRate, dev));
  const int grid = 2 * n_cu, waves = grid * 4;
  float* out = nullptr;
  unsigned long long* ticks = nullptr;
  CK(hipMalloc(&out, (size_t)grid * 256 * sizeof(float)));
  CK(hipMalloc(&ticks, (size_t)waves * 2 * sizeof(unsigned long long)));
  hipEvent_t e0, e1;
  CK(hipEventCreate(&e0));
  CK(hipEventCreate(&e1));
  mfma_kernel<<<grid, 256>>>(iters, out, ticks);   // warm-up
  CK(hipGetLastError());
  CK(hipDeviceSynchronize());
  const int reps = 5;
  CK(hipEventRecord(e0));
  for (int r = 0; r < reps; ++r) mfma_kernel<<<grid, 256>>>(iters, out, ticks);
  CK(hipEventRecord(e1));
  CK(hipEventSynchronize(e1));
  float ms = 0.f;
  CK(hipEventElapsedTime(&ms, e0, e1));
  unsigned long long* h = (unsigned long long*)malloc((size_t)waves * 2 * sizeof(unsigned long long));
  if (!h) return 1;
  CK(hipMemcpy(h, ticks, (size_t)waves * 2 * sizeof(unsigned long long), hipMemcpyDeviceToHost));
  double ghz = 0.0;
  // shader cycles per constant-clock tick, times that clock's rate
  for (int w = 0; w < waves; ++w) ghz += h[2 * w + 1] ? (double)h[2 * w] / (double)h[2 * w + 1] * wall_khz * 1e-6 : 0.0;
  ghz /= waves;
  const double us = ms * 1e3 / reps;
  const double flops = (double)waves * iters * kChains * 32.0 * 32.0 * 16.0 * 2.0;
  printf("{\"cus\": %d, \"workgroups\": %d, \"iters\": %d, \"us_per_launch\": %.2f, \"tflops\": %.1f, "
         "\"shader_ghz\": %.3f, \"wall_clock_khz\": %d}\n",
         n_cu, grid, iters, us, flops / (us * 1e-6) / 1e12, ghz, wall_khz);
  free(h);
  CK(hipFree(out));
  CK(hipFree(ticks));
  return 0;
}
