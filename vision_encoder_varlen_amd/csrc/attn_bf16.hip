// Varlen (block-diagonal) non-causal attention, bf16 in/out, for gfx950.
//
// Computes, for every work item (segment, q-tile) and head, the rows of
// softmax(Q K^T * scale) V restricted to the segment (vLLM page
// vllm.models.dots3_note.nvidia.vision_attention, VisionAttentionV2.forward;
// tokenspeed page mm_encoder_attention.py, vision_attn_fa3 with
// cu_seqlens_q = cu_seqlens_k).  The S x S mask of VisionAttention.forward is
// never formed: each workgroup only visits its own segment's keys.
//
// Design (one workgroup = 4 waves = 128 query rows of one head):
//  * Each wave owns 32 query rows.  Its Q fragments stay in VGPRs for the
//    whole key loop.
//  * Keys stream through LDS in tiles of 64, double-buffered: the global loads
//    of tile t+1 are issued before the math of tile t and written to the other
//    LDS buffer after it, so one barrier per tile suffices.
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: the query index then runs along the lanes, so
//    the row max and row sum of the online softmax are in-lane reductions plus
//    one exchange between the two 32-lane halves.
//  * K rows are stored in LDS with bits 2 and 3 of the key index swapped.
//    With that order the 32x32 accumulator layout hands each lane eight
//    consecutive keys per 16-key step, which is exactly the B operand layout of
//    the P V^T product, so P goes from the score registers to the next MFMA
//    without any cross-lane shuffle.
//  * O^T = V^T P^T is accumulated in fp32; V is transposed (4x4 blocks of
//    bf16 in registers) on its way into LDS so each MFMA A fragment is one
//    16-byte LDS read.
//  * Softmax runs in base 2 on fp32 scores with the scale folded into one
//    multiply: p = 2^(s*scale*log2(e) - m).
//  * LDS rows are padded by 16 bytes (an odd number of 16-byte slots per row),
//    so eight consecutive rows read at the same column hit distinct banks.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vit_kernels.h"

namespace vit {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned short u16;

constexpr int kBM = kBlockMBf16;  // query rows per workgroup
constexpr int kBN = 64;           // keys per LDS tile
constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;

template <int D>
struct Cfg {
  static constexpr int KSTEPS = D / 16;                 // 16-wide contraction steps of Q K^T
  static constexpr int DB = (D + 31) / 32;              // 32-row blocks of O^T
  static constexpr int DP = DB * 32;                    // head dim padded for the V^T tile
  static constexpr int KROW = D + 8;                    // K tile row stride (elements)
  static constexpr int VROW = kBN + 8;                  // V^T tile row stride (elements)
  static constexpr int K_ELEMS = kBN * KROW;
  static constexpr int V_ELEMS = DP * VROW;
  static constexpr int LDS_ELEMS = 2 * (K_ELEMS + V_ELEMS);
  static constexpr int KCH = kBN * D / 8;               // 16-byte chunks per K tile
  static constexpr int KCH_PT = (KCH + kThreads - 1) / kThreads;
  static constexpr int VUN = (kBN / 4) * (D / 4);       // 4 keys x 4 dims units per V tile
  static constexpr int VUN_PT = (VUN + kThreads - 1) / kThreads;
  static_assert(D % 16 == 0, "head dim must be a multiple of 16");
};

__device__ __forceinline__ int swap_bits_2_3(int x) {
  return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1);
}

__device__ __forceinline__ unsigned int pack_lo(unsigned int a, unsigned int b) {
  return (a & 0xffffu) | (b << 16);
}
__device__ __forceinline__ unsigned int pack_hi(unsigned int a, unsigned int b) {
  return (a >> 16) | (b & 0xffff0000u);
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void attn_bf16_kernel(
    const u16* __restrict__ q, const u16* __restrict__ k, const u16* __restrict__ v,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ items,
    const int32_t* __restrict__ meta, int H, float scale_log2, u16* __restrict__ out) {
  using C = Cfg<D>;
  __shared__ __align__(16) u16 smem[C::LDS_ELEMS];
  u16* const ks = smem;                    // [2][kBN][KROW], row p holds key swap_bits_2_3(p)
  u16* const vts = smem + 2 * C::K_ELEMS;  // [2][DP][VROW], V^T

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int half = lane >> 5;
  const size_t tok_stride = size_t(H) * D;

  // Rows D..DP-1 of the V^T tiles feed only output rows that are never
  // stored; keep them finite.
  if constexpr (C::DP != D) {
    for (int i = tid; i < 2 * (C::DP - D) * C::VROW; i += kThreads) {
      const int b = i / ((C::DP - D) * C::VROW);
      const int r = i - b * (C::DP - D) * C::VROW;
      vts[b * C::V_ELEMS + D * C::VROW + r] = 0;
    }
  }

  const int64_t nunits = int64_t(meta[0]) * H;
  for (int64_t unit = blockIdx.x; unit < nunits; unit += gridDim.x) {
    const int item = int(unit / H);
    const int h = int(unit - int64_t(item) * H);
    const int seg = items[2 * item];
    const int qt = items[2 * item + 1];
    const int start = cu[seg];
    const int len = cu[seg + 1] - start;
    const int qrow = qt * kBM + wave * 32 + l32;
    const u16* const kbase = k + size_t(start) * tok_stride + size_t(h) * D;
    const u16* const vbase = v + size_t(start) * tok_stride + size_t(h) * D;

    // Q^T fragments (B operand of S^T = K Q^T): lane holds 8 dims of its row.
    bf16x8_t qf[C::KSTEPS];
    if (qrow < len) {
      const u16* qp = q + size_t(start + qrow) * tok_stride + size_t(h) * D + half * 8;
#pragma unroll
      for (int s = 0; s < C::KSTEPS; ++s)
        qf[s] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(qp + s * 16));
    } else {
#pragma unroll
      for (int s = 0; s < C::KSTEPS; ++s) qf[s] = bf16x8_t{};
    }

    f32x16_t o[C::DB];
#pragma unroll
    for (int b = 0; b < C::DB; ++b) o[b] = f32x16_t{};
    float m_run = -INFINITY;  // running max of the scaled (log2-domain) scores
    float l_run = 0.f;        // this lane's partial row sum

    u32x4_t kreg[C::KCH_PT];
    u32x2_t vreg[C::VUN_PT][4];

    auto load_tile = [&](int kv0) {
#pragma unroll
      for (int i = 0; i < C::KCH_PT; ++i) {
        const int c = tid + i * kThreads;
        kreg[i] = u32x4_t{};
        if (c < C::KCH) {
          const int key = c / (D / 8);
          const int dc = c - key * (D / 8);
          if (kv0 + key < len)
            kreg[i] = *reinterpret_cast<const u32x4_t*>(kbase + size_t(kv0 + key) * tok_stride + dc * 8);
        }
      }
#pragma unroll
      for (int i = 0; i < C::VUN_PT; ++i) {
        const int u = tid + i * kThreads;
#pragma unroll
        for (int j = 0; j < 4; ++j) vreg[i][j] = u32x2_t{};
        if (u < C::VUN) {
          const int kq = u / (D / 4);
          const int dq = u - kq * (D / 4);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int key = kv0 + 4 * kq + j;
            if (key < len)
              vreg[i][j] = *reinterpret_cast<const u32x2_t*>(vbase + size_t(key) * tok_stride + dq * 4);
          }
        }
      }
    };

    auto store_tile = [&](int buf) {
      u16* kdst = ks + buf * C::K_ELEMS;
      u16* vdst = vts + buf * C::V_ELEMS;
#pragma unroll
      for (int i = 0; i < C::KCH_PT; ++i) {
        const int c = tid + i * kThreads;
        if (c < C::KCH) {
          const int key = c / (D / 8);
          const int dc = c - key * (D / 8);
          *reinterpret_cast<u32x4_t*>(kdst + swap_bits_2_3(key) * C::KROW + dc * 8) = kreg[i];
        }
      }
#pragma unroll
      for (int i = 0; i < C::VUN_PT; ++i) {
        const int u = tid + i * kThreads;
        if (u < C::VUN) {
          const int kq = u / (D / 4);
          const int dq = u - kq * (D / 4);
          u16* dst = vdst + (dq * 4) * C::VROW + kq * 4;
          const u32x2_t* r = vreg[i];
          // 4x4 transpose of bf16: row j = key 4kq+j, column e = dim 4dq+e.
          *reinterpret_cast<u32x2_t*>(dst + 0 * C::VROW) =
              u32x2_t{pack_lo(r[0].x, r[1].x), pack_lo(r[2].x, r[3].x)};
          *reinterpret_cast<u32x2_t*>(dst + 1 * C::VROW) =
              u32x2_t{pack_hi(r[0].x, r[1].x), pack_hi(r[2].x, r[3].x)};
          *reinterpret_cast<u32x2_t*>(dst + 2 * C::VROW) =
              u32x2_t{pack_lo(r[0].y, r[1].y), pack_lo(r[2].y, r[3].y)};
          *reinterpret_cast<u32x2_t*>(dst + 3 * C::VROW) =
              u32x2_t{pack_hi(r[0].y, r[1].y), pack_hi(r[2].y, r[3].y)};
        }
      }
    };

    const int ntiles = (len + kBN - 1) / kBN;
    load_tile(0);
    store_tile(0);
    __syncthreads();

    for (int t = 0; t < ntiles; ++t) {
      const int buf = t & 1;
      const int kv0 = t * kBN;
      if (t + 1 < ntiles) load_tile(kv0 + kBN);

      // S^T = K Q^T for 64 keys: two 32-key blocks.
      f32x16_t s[2];
      const u16* kt = ks + buf * C::K_ELEMS + l32 * C::KROW + half * 8;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = f32x16_t{};
#pragma unroll
        for (int st = 0; st < C::KSTEPS; ++st) {
          const bf16x8_t a = __builtin_bit_cast(
              bf16x8_t, *reinterpret_cast<const u32x4_t*>(kt + kb * 32 * C::KROW + st * 16));
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[st], s[kb], 0, 0, 0);
        }
      }

      // Online softmax.  Register r of block kb holds key
      // kv0 + 32kb + 16(r>>3) + 8half + (r&7) for query row l32.
      float mt = -INFINITY;
      const bool partial = kv0 + kBN > len;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = s[kb][r] * scale_log2;
          if (partial) {
            const int key = kv0 + kb * 32 + 16 * (r >> 3) + 8 * half + (r & 7);
            if (key >= len) x = -INFINITY;
          }
          s[kb][r] = x;
          mt = fmaxf(mt, x);
        }
      }
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      const float m_new = fmaxf(m_run, mt);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      float rsum = 0.f;
      bf16x8_t p[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = __builtin_amdgcn_exp2f(s[kb][r] - m_new);
          rsum += e;
          p[kb][r >> 3][r & 7] = (__bf16)e;
        }
      }
      l_run = l_run * alpha + rsum;
#pragma unroll
      for (int b = 0; b < C::DB; ++b) o[b] *= alpha;

      // O^T += V^T P^T.
      const u16* vt = vts + buf * C::V_ELEMS + l32 * C::VROW + half * 8;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
          for (int b = 0; b < C::DB; ++b) {
            const bf16x8_t a = __builtin_bit_cast(
                bf16x8_t,
                *reinterpret_cast<const u32x4_t*>(vt + b * 32 * C::VROW + kb * 32 + s2 * 16));
            o[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, p[kb][s2], o[b], 0, 0, 0);
          }
        }
      }

      if (t + 1 < ntiles) store_tile(buf ^ 1);
      __syncthreads();
    }

    // Finalize: O^T register r of block b holds dim 32b + 8(r>>2) + 4half + (r&3).
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float inv = 1.f / l_tot;
    if (qrow < len) {
      u16* op = out + size_t(start + qrow) * tok_stride + size_t(h) * D;
#pragma unroll
      for (int b = 0; b < C::DB; ++b) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d0 = b * 32 + 8 * g + 4 * half;
          if (d0 < D) {
            __bf16 w[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = (__bf16)(o[b][4 * g + e] * inv);
            *reinterpret_cast<u32x2_t*>(op + d0) = __builtin_bit_cast(u32x2_t, w);
          }
        }
      }
    }
    __syncthreads();  // LDS is reused by the next unit
  }
}

template <int D>
hipError_t launch_d(const void* q, const void* k, const void* v, const int32_t* cu,
                    const int32_t* items, int64_t cap, const int32_t* meta, int H, float scale,
                    void* out, hipStream_t stream) {
  int64_t units = cap * int64_t(H);
  if (units <= 0) return hipSuccess;
  const int64_t grid = units < kMaxAttnGrid ? units : kMaxAttnGrid;
  hipLaunchKernelGGL(attn_bf16_kernel<D>, dim3(unsigned(grid)), dim3(kThreads), 0, stream,
                     static_cast<const u16*>(q), static_cast<const u16*>(k),
                     static_cast<const u16*>(v), cu, items, meta, H, scale * kLog2e,
                     static_cast<u16*>(out));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bf16(const void* q, const void* k, const void* v, const int32_t* cu,
                            const int32_t* items, int64_t cap, const int32_t* meta, int H, int D,
                            float scale, void* out, hipStream_t stream) {
  switch (D) {
    case 32: return launch_d<32>(q, k, v, cu, items, cap, meta, H, scale, out, stream);
    case 64: return launch_d<64>(q, k, v, cu, items, cap, meta, H, scale, out, stream);
    case 80: return launch_d<80>(q, k, v, cu, items, cap, meta, H, scale, out, stream);
    case 96: return launch_d<96>(q, k, v, cu, items, cap, meta, H, scale, out, stream);
    case 128: return launch_d<128>(q, k, v, cu, items, cap, meta, H, scale, out, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace vit
