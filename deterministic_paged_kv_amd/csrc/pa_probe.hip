// Measurement kernels (include/pa_probe.h): a plain streaming read and a matrix-core loop, the
// measured ceilings the attention kernels' rates are reported against beside the published
// peaks.  Nothing here is part of the attention arithmetic.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_probe.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr uint32_t kNever = 0x9E3779B9u;  // a checksum value the probes treat as "never"

// Grid-stride read, four 16-byte loads in flight per thread before any is used.
__global__ __launch_bounds__(256) void probe_read_kernel(const uint4* __restrict__ src, size_t n16,
                                                         uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    acc ^= (a.x ^ b.y) + (c.z ^ d.w);
  }
  for (; i < n16; i += stride) {
    const uint4 a = src[i];
    acc ^= a.x + a.w;
  }
  if (acc == kNever) sink[blockIdx.x] = acc;
}

// Eight independent accumulation chains per wavefront; operands depend on the lane so the
// compiler cannot fold them.
template <int SHAPE>
__global__ __launch_bounds__(256) void probe_mfma_kernel(int iters, float* __restrict__ sink) {
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(float)((threadIdx.x + e) & 7);
    b[e] = (__bf16)(float)((threadIdx.x * 3 + e) & 7);
  }
  float s = 0.0f;
  if constexpr (SHAPE == 16) {
    f32x4 acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[c], 0, 0, 0);
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) s += acc[c][0] + acc[c][3];
  } else {
    f32x16 acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[c][e] = 0.0f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) s += acc[c][0] + acc[c][15];
  }
  if (__float_as_uint(s) == kNever) sink[blockIdx.x] = s;
}

}  // namespace

extern "C" {

int32_t pa_probe_read(const void* src, size_t bytes, int32_t blocks, void* sink, void* stream) {
  if (!src || !sink || bytes == 0 || bytes % 16 != 0 || ((uintptr_t)src & 15) != 0 || blocks < 1 ||
      blocks > 65536)
    return -1;
  hipLaunchKernelGGL(probe_read_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                     (const uint4*)src, bytes / 16, (uint32_t*)sink);
  return hipGetLastError() == hipSuccess ? 0 : -13;
}

int32_t pa_probe_mfma(int32_t blocks, int32_t iters, int32_t shape, void* sink, void* stream) {
  if (!sink || blocks < 1 || blocks > 65536 || iters < 1 || iters > (1 << 20) || (shape != 16 && shape != 32))
    return -1;
  if (shape == 16)
    hipLaunchKernelGGL(probe_mfma_kernel<16>, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, iters,
                       (float*)sink);
  else
    hipLaunchKernelGGL(probe_mfma_kernel<32>, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, iters,
                       (float*)sink);
  return hipGetLastError() == hipSuccess ? 0 : -13;
}

}  // extern "C"
