// Device work-list builder: cu_seqlens -> longest-first (segment, q-tile) items.
//
// The pages hand cu_seqlens and a caller-supplied max_seqlen straight to their
// varlen kernels (tokenspeed page mm_encoder_attention.py, _varlen_metadata);
// this list is the library's own schedule for the attention kernel.  Rule:
//   * len_i = cu[i+1] - cu[i]; validation sets sticky error bits and skips the
//     offending segment (bit 1: cu[0] != 0 -> empty list; bit 2: len_i < 0;
//     bit 4: len_i > max_seqlen; bit 8: capacity exceeded -> empty list);
//   * segments with len_i > 0 are ordered by len_i descending, ties by index
//     ascending (a unique order, so the list is bit-exact);
//   * each contributes (i, j) for j = 0 .. ceil(len_i / block_m) - 1.
// Attention workgroups are dispatched in list order, so the longest segments'
// tiles start first and the short ones fill the tail.
//
// One workgroup (one wave for up to 64 segments, up to 1024 threads for
// 8192) does everything in LDS, with no host sync:
// keys (len, index) are packed into 64-bit words so an ascending sort gives
// the order above; a sortedness check skips the bitonic network when the input
// is already ordered (uniform batches, single images); an exclusive scan of the
// per-segment tile counts (shuffles inside each wave, then the wave totals)
// gives each segment its slice of the list.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vit_kernels.h"
#include "worklist_build.h"

namespace vit {
namespace {

template <int THREADS>
__global__ __launch_bounds__(THREADS) void worklist_kernel(
    const int32_t* __restrict__ cu, int N, int npad, int max_seqlen, int block_m,
    int32_t* __restrict__ items, long long cap, int32_t* __restrict__ meta) {
  extern __shared__ __align__(16) unsigned long long keys[];  // [npad]
  int* const offs = reinterpret_cast<int*>(keys + npad);       // [npad] exclusive tile offsets
  __shared__ int s_wave[THREADS / 64];
  wl::build_worklist<THREADS>(cu, N, npad, max_seqlen, block_m, items, cap, meta, keys, offs, s_wave);
}

template <int THREADS>
hipError_t launch_t(const int32_t* cu, int N, int npad, int max_seqlen, int block_m,
                    int32_t* items, long long cap, int32_t* meta, hipStream_t stream,
                    hipEvent_t e0, hipEvent_t e1) {
  const size_t lds = size_t(npad) * (sizeof(unsigned long long) + sizeof(int));
  if (lds > 65536) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(worklist_kernel<THREADS>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    if (e != hipSuccess) return e;
  }
  hipExtLaunchKernelGGL(worklist_kernel<THREADS>, dim3(1), dim3(THREADS), lds, stream, e0, e1, 0,
                        cu, N, npad, max_seqlen, block_m, items, cap, meta);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_worklist(const int32_t* cu, int N, int max_seqlen, int block_m,
                           int32_t* items, int64_t cap, int32_t* meta, hipStream_t stream,
                           hipEvent_t e0, hipEvent_t e1) {
  int npad = 1;
  while (npad < N) npad <<= 1;
  // One wave for small batches (no cross-wave barriers on the critical path),
  // up to 1024 threads for large ones.
  if (npad <= 64) return launch_t<64>(cu, N, npad, max_seqlen, block_m, items, cap, meta, stream, e0, e1);
  if (npad <= 1024) return launch_t<256>(cu, N, npad, max_seqlen, block_m, items, cap, meta, stream, e0, e1);
  return launch_t<1024>(cu, N, npad, max_seqlen, block_m, items, cap, meta, stream, e0, e1);
}

}  // namespace vit
