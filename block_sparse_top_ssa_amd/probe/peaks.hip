// Peak microbenchmarks (declared in include/ssa_probe.h): the bf16 matrix-core issue rate
// and the HBM streaming-read rate of the device, for the roofline figures.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "ssa_probe.h"

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kChains = 8;  // independent accumulators per wave: products issue back to back

__global__ __launch_bounds__(256) void mfma_peak_kernel(int iters, float* __restrict__ out) {
  const uint32_t lane = threadIdx.x & 63;
  // bf16 operands near 1 (0x3F80) with a lane-dependent low mantissa bit
  const u32x4 a = {0x3F803F80u ^ (lane & 1), 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  const u32x4 b = {0x3F803F80u, 0x3F803F80u ^ ((lane >> 1) & 1), 0x3F803F80u, 0x3F803F80u};
  f32x4 acc[kChains];
#pragma unroll
  for (int u = 0; u < kChains; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Each product accumulates in place into its own AGPR quadruple (destination = C). With
  // the builtin the register allocator rotated the accumulators through copies at the
  // loop edge, and those copies waited on the products in flight.
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < kChains; ++u) asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc[u]) : "v"(a), "v"(b));
  }
  float s = 0.f;
#pragma unroll
  for (int u = 0; u < kChains; ++u) s += acc[u][0] + acc[u][1] + acc[u][2] + acc[u][3];
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

// Each workgroup reads a contiguous slice (measured faster than a grid-wide stride, whose
// concurrent accesses crowd the same memory channels), eight 16-byte loads in flight per
// thread.
__global__ __launch_bounds__(256) void hbm_read_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                       u32x4* __restrict__ out) {
  const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t b0 = (int64_t)blockIdx.x * per, b1 = b0 + per < n16 ? b0 + per : n16;
  int64_t i = b0 + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + 7 * 256 < b1; i += 8 * 256) {
    u32x4 x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) x[u] = src[i + u * 256];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= x[u];
  }
  for (; i < b1; i += 256) acc ^= src[i];
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

}  // namespace

extern "C" int ssa_probe_mfma_bf16(int blocks, int iters, float* out, void* stream) {
  if (blocks < 1 || iters < 1 || !out) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_peak_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, iters, out);
  return (int)hipGetLastError();
}

extern "C" int ssa_probe_hbm_read(const void* src, size_t bytes, int blocks, void* out, void* stream) {
  if (!src || !out || blocks < 1 || bytes % 16 || reinterpret_cast<uintptr_t>(src) % 16)
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(hbm_read_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                     static_cast<const u32x4*>(src), (int64_t)(bytes / 16), static_cast<u32x4*>(out));
  return (int)hipGetLastError();
}
