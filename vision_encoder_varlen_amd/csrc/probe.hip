// Sustained MFMA rate probe (measurement support; not part of the attention
// path).
//
// MI355X lowers its shader clock when MFMA operands toggle many bits, so the
// dense bf16 rate the chip sustains depends on the data.  This kernel issues
// nothing but v_mfma_f32_32x32x16_bf16 (four independent accumulator chains
// per wave) on operands read once from a caller buffer, so timing it with
// random operands and with zeros brackets what any bf16 MFMA kernel can reach
// on the same data.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vit_kernels.h"

namespace vit {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kProbeThreads) void probe_mfma_kernel(const u32x4_t* __restrict__ src,
                                                                   int iters, float* __restrict__ sink) {
  // 8 A and 8 B fragments per lane; block b reads slice b % kProbeSlices.
  const u32x4_t* p = src + (size_t(blockIdx.x % kProbeSlices) * kProbeThreads + threadIdx.x) * 16;
  bf16x8_t a[8], b[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = __builtin_bit_cast(bf16x8_t, p[i]);
    b[i] = __builtin_bit_cast(bf16x8_t, p[8 + i]);
  }
  f32x16_t c[4] = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(i + j) & 7], b[(i + 2 * j) & 7], c[j], 0, 0, 0);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += c[j][r];
  sink[size_t(blockIdx.x) * kProbeThreads + threadIdx.x] = s;
}

}  // namespace

hipError_t launch_probe_mfma(const void* operands, int blocks, int iters, float* sink,
                             hipStream_t stream) {
  hipLaunchKernelGGL(probe_mfma_kernel, dim3(unsigned(blocks)), dim3(kProbeThreads), 0, stream,
                     static_cast<const u32x4_t*>(operands), iters, sink);
  return hipGetLastError();
}

}  // namespace vit
