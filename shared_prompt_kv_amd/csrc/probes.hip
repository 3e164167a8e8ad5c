// Measurement probes for gfx950 (librelay_probes.so): a plain streaming read and a
// register-only matrix-core loop, the ceilings this GPU reaches at all.  Not part of
// the attention path.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/relay_probes.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kUnroll = 8;  // 16-byte loads in flight per thread

// Workgroup b reads 16-byte words [b per, min((b + 1) per, n16)): per iteration each
// thread issues kUnroll loads, kThreads words apart, before it consumes any.
__global__ __launch_bounds__(kThreads) void read_probe_kernel(const u32x4* buf, size_t n16, float* sink) {
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t b0 = (size_t)blockIdx.x * per;
  const size_t b1 = b0 + per < n16 ? b0 + per : n16;
  uint32_t acc = 0;
  for (size_t i = b0 + threadIdx.x; i < b1; i += (size_t)kThreads * kUnroll) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const size_t j = i + (size_t)u * kThreads;
      v[u] = j < b1 ? buf[j] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  __shared__ uint32_t red[kThreads];
  red[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t x = 0;
    for (int t = 0; t < kThreads; ++t) x ^= red[t];
    sink[blockIdx.x] = (float)(x & 0xffffu);
  }
}

// Four independent accumulators per wave, operands fixed in registers (bf16 1/64 and
// 1/32, so sums stay far from overflow).
__global__ __launch_bounds__(kThreads) void mfma_probe_kernel(int iters, float* sink) {
  const uint32_t a_bits = 0x3c80u | (0x3c80u << 16);  // bf16 1/64, twice
  const uint32_t b_bits = 0x3d00u | (0x3d00u << 16);  // bf16 1/32, twice
  const u32x4 a = {a_bits, a_bits, a_bits, a_bits};
  const u32x4 b = {b_bits, b_bits, b_bits, b_bits};
  f32x16 acc[4] = {f32x16{}, f32x16{}, f32x16{}, f32x16{}};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < 4; ++k)
      acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                       acc[k], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int j = 0; j < 16; ++j) s += acc[k][j];
  sink[(size_t)blockIdx.x * kThreads + threadIdx.x] = s;
}

}  // namespace

extern "C" {

int relay_probe_read(const void* buf, size_t bytes, float* sink, int32_t workgroups, void* stream) {
  if (!buf || !sink || bytes == 0 || bytes % 16 != 0 || ((uintptr_t)buf & 15u) != 0 || workgroups < 1) return -1;
  hipLaunchKernelGGL(read_probe_kernel, dim3(workgroups), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(buf), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int relay_probe_mfma(float* sink, int32_t iters, int32_t workgroups, void* stream) {
  if (!sink || iters < 1 || workgroups < 1) return -1;
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(workgroups), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     (int)iters, sink);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // extern "C"
