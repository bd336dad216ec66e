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
// One workgroup of 1024 threads does everything in LDS, with no host sync:
// keys (len, index) are packed into 64-bit words so an ascending sort gives
// the order above; a sortedness check skips the bitonic network when the input
// is already ordered (uniform batches, single images); an exclusive scan of the
// per-segment tile counts gives each segment its slice of the list.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vit_kernels.h"

namespace vit {
namespace {

constexpr int kThreads = 1024;
constexpr unsigned long long kEmpty = ~0ull;

__global__ __launch_bounds__(kThreads) void worklist_kernel(
    const int32_t* __restrict__ cu, int N, int npad, int max_seqlen, int block_m,
    int32_t* __restrict__ items, long long cap, int32_t* __restrict__ meta) {
  extern __shared__ __align__(16) unsigned long long keys[];  // [npad]
  int* const offs = reinterpret_cast<int*>(keys + npad);       // [npad] exclusive tile offsets
  __shared__ int s_err;
  __shared__ int s_unsorted;
  __shared__ int s_partial[kThreads];

  const int tid = threadIdx.x;
  if (tid == 0) {
    s_err = (N > 0 && cu[0] != 0) ? 1 : 0;
    s_unsorted = 0;
  }
  __syncthreads();
  const bool cu0_bad = s_err & 1;

  // 1. keys: high word = 0x7fffffff - len (ascending = longest first), low = index.
  for (int i = tid; i < npad; i += kThreads) {
    unsigned long long key = kEmpty;
    if (i < N && !cu0_bad) {
      const int len = cu[i + 1] - cu[i];
      if (len < 0) {
        atomicOr(&s_err, 2);
      } else if (len > max_seqlen) {
        atomicOr(&s_err, 4);
      } else if (len > 0) {
        key = (static_cast<unsigned long long>(0x7fffffffu - static_cast<unsigned>(len)) << 32) |
              static_cast<unsigned>(i);
      }
    }
    keys[i] = key;
  }
  __syncthreads();

  // 2. sort only when needed.
  for (int i = tid; i + 1 < npad; i += kThreads)
    if (keys[i] > keys[i + 1]) s_unsorted = 1;
  __syncthreads();
  if (s_unsorted) {
    for (int size = 2; size <= npad; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int i = tid; i < npad; i += kThreads) {
          const int j = i ^ stride;
          if (j > i) {
            const unsigned long long a = keys[i], b = keys[j];
            const bool ascending = (i & size) == 0;
            if ((a > b) == ascending) {
              keys[i] = b;
              keys[j] = a;
            }
          }
        }
        __syncthreads();
      }
    }
  }

  // 3. exclusive scan of tile counts: each thread owns a contiguous chunk.
  const int chunk = (npad + kThreads - 1) / kThreads;
  const int c0 = tid * chunk;
  int local = 0;
  for (int i = c0; i < c0 + chunk && i < npad; ++i) {
    const unsigned long long key = keys[i];
    int nt = 0;
    if (key != kEmpty) {
      const int len = int(0x7fffffffu - static_cast<unsigned>(key >> 32));
      nt = (len + block_m - 1) / block_m;
    }
    offs[i] = nt;
    local += nt;
  }
  s_partial[tid] = local;
  __syncthreads();
  for (int d = 1; d < kThreads; d <<= 1) {  // inclusive Hillis-Steele scan of partials
    const int add = tid >= d ? s_partial[tid - d] : 0;
    __syncthreads();
    s_partial[tid] += add;
    __syncthreads();
  }
  int run = s_partial[tid] - local;  // exclusive prefix of this chunk
  for (int i = c0; i < c0 + chunk && i < npad; ++i) {
    const int nt = offs[i];
    offs[i] = run;
    run += nt;
  }
  const int total = s_partial[kThreads - 1];
  __syncthreads();

  // 4. scatter.
  const bool overflow = static_cast<long long>(total) > cap;
  if (!overflow) {
    for (int i = tid; i < npad; i += kThreads) {
      const unsigned long long key = keys[i];
      if (key == kEmpty) continue;
      const int seg = int(key & 0xffffffffu);
      const int len = int(0x7fffffffu - static_cast<unsigned>(key >> 32));
      const int nt = (len + block_m - 1) / block_m;
      const int base = offs[i];
      for (int j = 0; j < nt; ++j) {
        items[2 * (base + j)] = seg;
        items[2 * (base + j) + 1] = j;
      }
    }
  }
  if (tid == 0) {
    meta[0] = overflow ? 0 : total;
    meta[1] = s_err | (overflow ? 8 : 0);
  }
}

}  // namespace

hipError_t launch_worklist(const int32_t* cu, int N, int max_seqlen, int block_m,
                           int32_t* items, int64_t cap, int32_t* meta, hipStream_t stream,
                           hipEvent_t e0, hipEvent_t e1) {
  int npad = 1;
  while (npad < N) npad <<= 1;
  const size_t lds = size_t(npad) * (sizeof(unsigned long long) + sizeof(int));
  if (lds > 65536) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(worklist_kernel),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    if (e != hipSuccess) return e;
  }
  hipExtLaunchKernelGGL(worklist_kernel, dim3(1), dim3(kThreads), lds, stream, e0, e1, 0, cu, N, npad,
                     max_seqlen, block_m, items, static_cast<long long>(cap), meta);
  return hipGetLastError();
}

}  // namespace vit
