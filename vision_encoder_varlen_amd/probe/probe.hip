// Sustained MFMA rate probe: measurement support, built as its own library
// (libvit_probe.so) and not part of the attention path or of libvit.so.
//
// MI355X lowers its shader clock when MFMA operands toggle many bits, so the
// dense bf16 rate the chip sustains depends on the data.  This kernel issues
// nothing but v_mfma_f32_32x32x16_bf16 (four independent accumulator chains
// per wave) on operands read once from a caller buffer, so timing it with
// random operands and with zeros brackets what any bf16 MFMA kernel can reach
// on the same data.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>

#include "vit_probe.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// Workgroups of kThreads threads; each lane reads 256 operand bytes from
// slice blockIdx % kSlices, so the operands span kOperandBytes.
constexpr int kThreads = 256;
constexpr int kSlices = 64;
constexpr int64_t kOperandBytes = int64_t(kSlices) * kThreads * 256;

__global__ __launch_bounds__(kThreads) void probe_mfma_kernel(const u32x4_t* __restrict__ src, int iters,
                                                              float* __restrict__ sink) {
  // 8 A and 8 B fragments per lane; block b reads slice b % kSlices.
  const u32x4_t* p = src + (size_t(blockIdx.x % kSlices) * kThreads + threadIdx.x) * 16;
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
  sink[size_t(blockIdx.x) * kThreads + threadIdx.x] = s;
}

thread_local char g_err[256];

int fail(int code, const char* msg) {
  snprintf(g_err, sizeof(g_err), "%s", msg);
  return code;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

}  // namespace

extern "C" {

int vit_probe_mfma(const void* operands, int64_t operand_bytes, int blocks, int iters, float* sink,
                   hipStream_t stream) {
  if (!operands || !sink) return fail(1, "null pointer argument");
  if (operand_bytes < kOperandBytes) return fail(1, "operands must hold 4 MiB (4194304 bytes)");
  if (!aligned(operands, 16) || !aligned(sink, 4)) return fail(1, "misaligned buffer");
  if (blocks < 1 || blocks > 65536 || iters < 1 || iters > (1 << 20))
    return fail(1, "blocks in [1, 65536] and iters in [1, 2^20] required");
  hipLaunchKernelGGL(probe_mfma_kernel, dim3(unsigned(blocks)), dim3(kThreads), 0, stream,
                     static_cast<const u32x4_t*>(operands), iters, sink);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(3, hipGetErrorString(e));
  g_err[0] = '\0';
  return 0;
}

const char* vit_probe_last_error(void) { return g_err; }

}  // extern "C"
