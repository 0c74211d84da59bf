// Measurement probe used by bench.py (libiha_probe.so, not part of the forward pass): the
// dense fp16 matrix-core rate this chip sustains under a pure-product load, and the shader
// clock it runs at meanwhile.  The datasheet peak (2.5 PFLOP/s) assumes 2.4 GHz; under
// sustained matrix-core load the clock drops, and this gives the figure to read the
// kernels' roofline fractions against.
#include "iha_probe.h"

#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;  // 4 waves per workgroup
constexpr int kChains = 4;     // independent accumulators per wave
constexpr int kPerIter = 16;   // products per loop iteration

// Every wave issues iters * kPerIter independent 32x32x16 fp16 products (32768 flops each).
// Wave 0 of workgroup 0 records the shader-clock counter (s_memtime) and the constant
// 100 MHz counter (s_memrealtime) around its loop.  The accumulated values are written to
// `sink` only if they take an impossible value, so the products are not removed.
__global__ __launch_bounds__(kThreads) void mfma_rate_kernel(int iters, float* sink, int64_t* stamps) {
  half8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = static_cast<_Float16>((threadIdx.x & 63) * 1e-3f + e * 1e-2f);
    b[e] = static_cast<_Float16>(e * 0.5f);
  }
  floatx16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
  const bool rec = blockIdx.x == 0 && threadIdx.x == 0;
  int64_t t0 = 0, r0 = 0;
  if (rec) {
    t0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < kPerIter; ++i)
      acc[i % kChains] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[i % kChains], 0, 0, 0);
  }
  if (rec) {
    const int64_t t1 = __builtin_amdgcn_s_memtime();
    const int64_t r1 = __builtin_amdgcn_s_memrealtime();
    stamps[0] = t1 - t0;
    stamps[1] = r1 - r0;
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  if (s == -12345.f) sink[blockIdx.x * kThreads + threadIdx.x] = s;
}

}  // namespace

extern "C" int ihp_mfma_rate(int milliseconds, double* tflops, double* clock_mhz, double* kernel_ms) {
  if (milliseconds < 1 || !tflops || !clock_mhz || !kernel_ms) return 1;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 2;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) return 2;
  const int blocks = cus * 2;  // two workgroups per CU: two waves per SIMD
  float* sink = nullptr;
  int64_t* stamps = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  int rc = 0;
  if (hipMalloc(&sink, sizeof(float) * blocks * kThreads) != hipSuccess ||
      hipMalloc(&stamps, 2 * sizeof(int64_t)) != hipSuccess || hipEventCreate(&e0) != hipSuccess ||
      hipEventCreate(&e1) != hipSuccess) {
    rc = 2;
  } else {
    // A short run sizes the iteration count for the requested duration; a full-length run
    // brings the clocks to their sustained level; the third is the one timed.
    int iters = 2000;
    float ms = 0.f;
    for (int pass = 0; pass < 3 && rc == 0; ++pass) {
      hipEventRecord(e0, nullptr);
      hipLaunchKernelGGL(mfma_rate_kernel, dim3(blocks), dim3(kThreads), 0, nullptr, iters, sink, stamps);
      hipEventRecord(e1, nullptr);
      if (hipEventSynchronize(e1) != hipSuccess || hipEventElapsedTime(&ms, e0, e1) != hipSuccess) rc = 3;
      if (pass == 0 && rc == 0 && ms > 0.f) {
        const double scaled = iters * (milliseconds / static_cast<double>(ms));
        iters = static_cast<int>(scaled < 2e6 ? (scaled > 100 ? scaled : 100) : 2e6);  // <= ~1 s
      }
    }
    int64_t h[2] = {0, 0};
    if (rc == 0 && hipMemcpy(h, stamps, sizeof(h), hipMemcpyDeviceToHost) != hipSuccess) rc = 3;
    if (rc == 0) {
      const double flops = static_cast<double>(blocks) * (kThreads / 64) * iters * kPerIter * 32768.0;
      *tflops = flops / (ms * 1e-3) / 1e12;
      *clock_mhz = h[1] > 0 ? 100.0 * static_cast<double>(h[0]) / static_cast<double>(h[1]) : 0.0;
      *kernel_ms = ms;
    }
  }
  if (e0) hipEventDestroy(e0);
  if (e1) hipEventDestroy(e1);
  if (sink) hipFree(sink);
  if (stamps) hipFree(stamps);
  return rc;
}
