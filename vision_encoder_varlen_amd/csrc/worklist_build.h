// Work-list build, shared by the work-list kernel and the fused pre-pass +
// work-list launch.  The rule and the algorithm are described in
// worklist.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vit {
namespace wl {

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

// Builds the list with THREADS threads of one workgroup.  keys and offs are
// LDS arrays of npad entries (npad = next power of two >= N), s_wave an LDS
// array of THREADS / 64 ints.  Item i is four int32 at items + 4i:
// (segment, q-tile, first token cu[segment], length); items
// [count, min(cap, count + kWorklistSentinelSpan)) get segment -1, so an
// attention workgroup can read its item without first reading the count.
template <int THREADS>
__device__ __forceinline__ void build_worklist(const int32_t* __restrict__ cu, int N, int npad,
                                               int max_seqlen, int block_m,
                                               int32_t* __restrict__ items, long long cap,
                                               int32_t* __restrict__ meta,
                                               unsigned long long* keys, int* offs, int* s_wave) {
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
      const int first = cu[seg];
      for (int j = 0; j < nt; ++j)
        *reinterpret_cast<int4*>(items + 4 * (long long)(base + j)) = make_int4(seg, j, first, len);
    }
  }
  // Sentinels after the last item (from the start when the list is empty).
  {
    const long long from = overflow ? 0 : static_cast<long long>(total);
    const long long to = from + kWorklistSentinelSpan < cap ? from + kWorklistSentinelSpan : cap;
    for (long long i = from + tid; i < to; i += THREADS)
      *reinterpret_cast<int4*>(items + 4 * i) = make_int4(-1, 0, 0, 0);
  }
  if (tid == 0) {
    meta[0] = overflow ? 0 : total;
    meta[1] = (cu0_bad ? 1 : 0) | err_any | err_long | (overflow ? 8 : 0);
  }
}

}  // namespace wl
}  // namespace vit
