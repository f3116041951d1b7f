// Attainable-peak probes (measurement aids, not part of the operator): a
// bf16 matrix-core loop and a streaming device copy.  They give what the chip
// sustains under load, to set beside its published peaks when a kernel's
// fraction of the roofline is reported.
#include "common.h"

namespace up {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Every wave runs `iters` rounds of four independent 32x32x16 bf16 products
// (32768 flops each) on operands with varied bits (data-dependent power
// is part of what a real kernel sees), then folds its accumulators into
// sink[thread] so nothing is dead code.
__global__ __launch_bounds__(256) void peak_mfma_kernel(int iters, float* __restrict__ sink) {
  const int tid = blockIdx.x * 256 + threadIdx.x;
  uint32_t h = (uint32_t)tid * 2654435761u + 12345u;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    h = h * 1664525u + 1013904223u;
    a[e] = (__bf16)((float)((int)((h >> 12) & 1023) - 512) * (1.0f / 512.0f));
    h = h * 1664525u + 1013904223u;
    b[e] = (__bf16)((float)((int)((h >> 12) & 1023) - 512) * (1.0f / 4096.0f));
  }
  f32x16 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[j][e];
  sink[tid] = s;
}

// Each workgroup copies 32 KiB chunks (eight 16-byte non-temporal loads in
// flight per thread, then eight stores), chunks strided by the grid; the
// tail past the last whole chunk goes one 16-byte word per thread.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kCopyUnroll = 8;
__global__ __launch_bounds__(256) void peak_copy_kernel(const u32x4* __restrict__ src,
                                                        u32x4* __restrict__ dst, long n16) {
  const long chunk = (long)kCopyUnroll * 256;
  const long nch = n16 / chunk;
  for (long c = blockIdx.x; c < nch; c += gridDim.x) {
    const long b = c * chunk + threadIdx.x;
    u32x4 x[kCopyUnroll];
#pragma unroll
    for (int j = 0; j < kCopyUnroll; ++j) x[j] = __builtin_nontemporal_load(src + b + j * 256);
#pragma unroll
    for (int j = 0; j < kCopyUnroll; ++j) __builtin_nontemporal_store(x[j], dst + b + j * 256);
  }
  for (long i = nch * chunk + (long)blockIdx.x * 256 + threadIdx.x; i < n16;
       i += (long)gridDim.x * 256)
    dst[i] = src[i];
}

hipError_t launch_peak_mfma(int workgroups, int iters, float* sink, hipStream_t st) {
  hipLaunchKernelGGL(peak_mfma_kernel, dim3(workgroups), dim3(256), 0, st, iters, sink);
  return hipGetLastError();
}

hipError_t launch_peak_copy(const void* src, void* dst, size_t bytes, hipStream_t st) {
  const long n16 = (long)(bytes / 16);
  hipLaunchKernelGGL(peak_copy_kernel, dim3(4096), dim3(256), 0, st, (const u32x4*)src,
                     (u32x4*)dst, n16);
  return hipGetLastError();
}

}  // namespace up
