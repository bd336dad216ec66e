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

namespace vit {
namespace {

constexpr unsigned long long kEmpty = ~0ull;

// Exclusive prefix over the workgroup of one int per thread, plus the total:
// a shuffle scan inside each wave, then the wave totals through LDS (one
// barrier).
template <int THREADS>
__device__ __forceinline__ int block_exclusive_scan(int v, int* s_wave, int* total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(incl, d);
    if (lane >= d) incl += y;
  }
  if (lane == 63) s_wave[wave] = incl;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < THREADS / 64; ++w) {
    const int t = s_wave[w];
    before += w < wave ? t : 0;
    all += t;
  }
  *total = all;
  return before + incl - v;
}

template <int THREADS>
__global__ __launch_bounds__(THREADS) void worklist_kernel(
    const int32_t* __restrict__ cu, int N, int npad, int max_seqlen, int block_m,
    int32_t* __restrict__ items, long long cap, int32_t* __restrict__ meta) {
  extern __shared__ __align__(16) unsigned long long keys[];  // [npad]
  int* const offs = reinterpret_cast<int*>(keys + npad);       // [npad] exclusive tile offsets
  __shared__ int s_wave[THREADS / 64];

  const int tid = threadIdx.x;
  // Every thread reads cu[0] with its own entries: one round trip to memory.
  const bool cu0_bad = N > 0 && cu[0] != 0;
  int err = cu0_bad ? 1 : 0;

  // 1. keys: high word = 0x7fffffff - len (ascending = longest first), low = index.
  for (int i = tid; i < npad; i += THREADS) {
    unsigned long long key = kEmpty;
    if (i < N && !cu0_bad) {
      const int len = cu[i + 1] - cu[i];
      if (len < 0) {
        err |= 2;
      } else if (len > max_seqlen) {
        err |= 4;
      } else if (len > 0) {
        key = (static_cast<unsigned long long>(0x7fffffffu - static_cast<unsigned>(len)) << 32) |
              static_cast<unsigned>(i);
      }
    }
    keys[i] = key;
  }
  const int err_any = __syncthreads_or(err & 2) ? 2 : 0;
  const int err_long = __syncthreads_or(err & 4) ? 4 : 0;

  // 2. sort only when needed.
  int unsorted = 0;
  for (int i = tid; i + 1 < npad; i += THREADS)
    if (keys[i] > keys[i + 1]) unsorted = 1;
  if (__syncthreads_or(unsorted)) {
    for (int size = 2; size <= npad; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int i = tid; i < npad; i += THREADS) {
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
  const int chunk = (npad + THREADS - 1) / THREADS;
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
  int total = 0;
  int run = block_exclusive_scan<THREADS>(local, s_wave, &total);
  for (int i = c0; i < c0 + chunk && i < npad; ++i) {
    const int nt = offs[i];
    offs[i] = run;
    run += nt;
  }

  // 4. scatter (each thread reads back only the offsets it wrote).
  const bool overflow = static_cast<long long>(total) > cap;
  if (!overflow) {
    for (int i = c0; i < c0 + chunk && i < npad; ++i) {
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
    meta[1] = (cu0_bad ? 1 : 0) | err_any | err_long | (overflow ? 8 : 0);
  }
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
