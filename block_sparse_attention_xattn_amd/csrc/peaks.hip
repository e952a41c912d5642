// Peak-rate microbenchmarks for gfx950 (libxattn_peaks.so): the references the
// bench reports next to the published peaks. Measurement code only; the
// attention library does not use it.
//
//  * matrix-core rate: every wave issues v_mfma_f32_32x32x16_bf16 on four
//    independent accumulators (no memory traffic), two waves per SIMD;
//  * sustained core clock under that load: per workgroup, the core-clock
//    counter (s_memtime) against the 100 MHz reference counter
//    (s_memrealtime) over the same interval;
//  * HBM stream copy: 16-byte vector loads and stores, grid-stride.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/xattn_peaks.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;  // per workgroup: two per SIMD

__global__ __launch_bounds__(64 * kWaves) void mfma_loop_kernel(int iters, float* sink,
                                                               unsigned long long* clk) {
  const int tid = threadIdx.x;
  unsigned long long t0 = 0, r0 = 0;
  if (clk && tid == 0) {
    t0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = static_cast<__bf16>(1e-3f * (float)((tid + i) & 7));
    b[i] = static_cast<__bf16>(1e-3f * (float)i);
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  sink[blockIdx.x * blockDim.x + tid] = s;  // keeps the loop alive
  if (clk && tid == 0) {
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    clk[2 * blockIdx.x] = t1 - t0;
    clk[2 * blockIdx.x + 1] = r1 - r0;
  }
}

__global__ __launch_bounds__(256) void copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                   size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

}  // namespace

extern "C" {

int32_t xattn_peak_mfma_waves_per_block(void) { return kWaves; }

int32_t xattn_peak_mfma(int32_t blocks, int32_t iters, float* sink, unsigned long long* clk, void* stream) {
  if (blocks < 1 || iters < 1 || !sink) return (int32_t)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(blocks), dim3(64 * kWaves), 0, static_cast<hipStream_t>(stream),
                     iters, sink, clk);
  return (int32_t)hipGetLastError();
}

int32_t xattn_peak_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (!src || !dst || bytes % 16 || bytes == 0) return (int32_t)hipErrorInvalidValue;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                              hipSuccess)
    return (int32_t)hipErrorInvalidDevice;
  hipLaunchKernelGGL(copy_kernel, dim3(cus * 8), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), bytes / 16);
  return (int32_t)hipGetLastError();
}

}  // extern "C"
