// mfma_clock.hip -- measurement probe (not part of libmoe): sustained shader
// clock and dense bf16 MFMA rate of MI355X under a pure MFMA load.
//
// Every wave issues back-to-back 32x32x16 bf16 MFMAs on register operands (no
// memory traffic) and reads s_memtime (counts shader clock cycles) and
// s_memrealtime (fixed-rate reference, hipDeviceAttributeWallClockRate) at its
// start and end; their ratio is the clock the waves actually ran at.  It is the
// reference for the counter method used on the library's kernels: rocprofv3's
// SQ_CYCLES / 32 (shader engines) / kernel duration gives the same figure for
// this kernel, so it gives the sustained clock of any kernel.
//
//   hipcc -O3 --offload-arch=gfx950 -Xclang -target-feature -Xclang -packed-fp32-ops \
//       sparse_mixture_experts_wavefront_amd/csrc/probe/mfma_clock.hip -o mfma_clock
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <stdint.h>
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void k(int iters, float* out, unsigned long long* clk) {
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) { a[i] = (__bf16)(0.001f * (threadIdx.x + i)); b[i] = (__bf16)(0.002f * i); }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  unsigned long long t0 = __builtin_amdgcn_s_memtime();
  unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  unsigned long long t1 = __builtin_amdgcn_s_memtime();
  unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  out[blockIdx.x * 256 + threadIdx.x] = s;
  if (threadIdx.x == 0) {
    clk[blockIdx.x * 2] = t1 - t0;
    clk[blockIdx.x * 2 + 1] = r1 - r0;
  }
}

#define CHECK(x)                                                        \
  do {                                                                  \
    hipError_t e_ = (x);                                                \
    if (e_ != hipSuccess) {                                             \
      printf("%s failed: %s\n", #x, hipGetErrorString(e_));              \
      return 1;                                                         \
    }                                                                   \
  } while (0)

int main() {
  int dev = 0, cus = 0, wall_khz = 0;
  CHECK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
  CHECK(hipDeviceGetAttribute(&wall_khz, hipDeviceAttributeWallClockRate, dev));
  const int blocks = cus * 4;   // 4 waves per SIMD
  const int iters = 20000;
  float* out;
  unsigned long long* clk;
  CHECK(hipMalloc(&out, (size_t)blocks * 256 * 4));
  CHECK(hipMalloc(&clk, (size_t)blocks * 16));
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  hipLaunchKernelGGL(k, dim3(blocks), dim3(256), 0, 0, 100, out, clk);  // warm-up
  CHECK(hipDeviceSynchronize());
  unsigned long long* h = (unsigned long long*)malloc((size_t)blocks * 16);
  for (int rep = 0; rep < 3; ++rep) {
    CHECK(hipEventRecord(e0, 0));
    hipLaunchKernelGGL(k, dim3(blocks), dim3(256), 0, 0, iters, out, clk);
    CHECK(hipEventRecord(e1, 0));
    CHECK(hipEventSynchronize(e1));
    float ms = 0;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    CHECK(hipMemcpy(h, clk, (size_t)blocks * 16, hipMemcpyDeviceToHost));
    double sc = 0, sr = 0;
    for (int b = 0; b < blocks; ++b) { sc += h[2 * b]; sr += h[2 * b + 1]; }
    const double mhz = sc / sr * (wall_khz / 1000.0);
    const double flops = (double)blocks * 4 /*waves*/ * iters * 4 * 32.0 * 32 * 16 * 2;
    printf("CUs %d wall_clock %d kHz: kernel %.3f ms, %.1f TFLOP/s bf16 MFMA, sustained shader clock %.0f MHz\n",
           cus, wall_khz, ms, flops / (ms * 1e-3) / 1e12, mhz);
  }
  free(h);
  return 0;
}
