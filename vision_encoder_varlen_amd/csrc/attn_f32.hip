// Varlen (block-diagonal) attention in fp32 throughout, non-causal or causal.
//
// Same operation as the bf16 kernel of attn_bf16_kernel.h (vLLM page
// vllm.models.dots3_note.nvidia.vision_attention, VisionAttentionV2.forward),
// for fp32 tensors where an exact-precision result is wanted.  No MFMA and no
// down-conversion: products and sums are fp32 FMAs and the softmax uses the
// accurate expf.
//
// One workgroup = one wave = 32 query rows of one head.  Lanes l and l+32 share
// query row l: each holds half of the head dim of q and of the output
// accumulator, and the two partial dot products are joined with one lane
// exchange, so both lanes see bit-identical scores.  Keys stream through LDS in
// tiles of 32 rows with a per-key online softmax.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "vit_kernels.h"

namespace vit {
namespace {

constexpr int kBM = kBlockMF32;
constexpr int kBN = 32;
constexpr int kThreads = 64;

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void attn_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ items,
    const int32_t* __restrict__ meta, int u_batch, int u_seq_len, int H, float scale,
    float* __restrict__ out, float* __restrict__ lse, TokenStrides ts, QPrepass qpre) {
  constexpr int HD = D / 2;
  constexpr int ROW = D + 4;  // +16 bytes per LDS row
  __shared__ __align__(16) float ks[kBN * ROW];
  __shared__ __align__(16) float vs[kBN * ROW];

  const int lane = threadIdx.x;
  const int r = lane & 31;
  const int half = lane >> 5;

  // items == null: a uniform batch (u_batch segments of u_seq_len tokens).
  const bool uniform = items == nullptr;
  const int uni_tiles = (u_seq_len + kBM - 1) / kBM;
  const int64_t nunits = (uniform ? int64_t(u_batch) * uni_tiles : int64_t(meta[0])) * H;
  for (int64_t unit = blockIdx.x; unit < nunits; unit += gridDim.x) {
    const int item = int(unit / H);
    const int h = int(unit - int64_t(item) * H);
    int qt, start, len;
    if (uniform) {
      const int seg = item / uni_tiles;
      qt = item - seg * uni_tiles;
      start = seg * u_seq_len;
      len = u_seq_len;
    } else {
      const int4 it = *reinterpret_cast<const int4*>(items + 4 * size_t(item));
      qt = it.y;
      start = it.z;
      len = it.w;
    }
    const int qrow = qt * kBM + r;

    float qv[HD], acc[HD];
#pragma unroll
    for (int d = 0; d < HD; ++d) acc[d] = 0.f;
    if (qrow < len) {
      const float* qp = q + size_t(start + qrow) * ts.q + size_t(h) * D + half * HD;
#pragma unroll
      for (int d = 0; d < HD; d += 4) {
        const float4 x = *reinterpret_cast<const float4*>(qp + d);
        qv[d] = x.x; qv[d + 1] = x.y; qv[d + 2] = x.z; qv[d + 3] = x.w;
      }
    } else {
#pragma unroll
      for (int d = 0; d < HD; ++d) qv[d] = 0.f;
    }
    // Pre-pass on one row held by a lane pair (RMSNorm with `weight`, then
    // rotary at `pr`; fp32).  This lane holds dims half * D/2 + d: rotate-half
    // partners sit in the other half of the wave at the same d; complex
    // partners are d ^ 1 in this lane.  Used for the query row, and with
    // fuse_k for each key row of a tile.
    auto prep_row = [&](float (&xv)[HD], const float* weight, int2 pr) {
      if (weight != nullptr) {
        float ss = 0.f;
#pragma unroll
        for (int d = 0; d < HD; ++d) ss = fmaf(xv[d], xv[d], ss);
        ss += __shfl_xor(ss, 32);
        const float rinv = rsqrtf(ss * (1.f / D) + qpre.eps);
#pragma unroll
        for (int d = 0; d < HD; ++d) xv[d] = xv[d] * rinv * weight[half * HD + d];
      }
      if (qpre.pos != nullptr) {
        // Angle of frequency F on the row (col = false) or column axis:
        // 2*pi * coord * rev[F], reduced to a fraction of a turn exactly, then
        // an accurate sincosf.  F is a compile-time constant (no dynamic
        // indexing of the parameter block).
        auto cos_sin = [&](auto f_c, bool col) {
          constexpr int F = decltype(f_c)::value;
          const float c = float(col ? pr.y : pr.x);
          const float t = c * qpre.rev_hi[F];
          const float frac = (t - rintf(t)) + (fmaf(c, qpre.rev_hi[F], -t) + c * qpre.rev_lo[F]);
          float sn, cn;
          sincosf(6.283185307179586f * frac, &sn, &cn);
          return make_float2(cn, sn);
        };
        if (qpre.rope_mode == 0) {
          // pair index j = d for both halves
          static_for<HD>([&](auto d_c) {
            constexpr int d = decltype(d_c)::value;
            const float part = __shfl_xor(xv[d], 32);
            const float2 cs = cos_sin(std::integral_constant<int, (d < D / 4 ? d : d - D / 4)>{},
                                      d >= D / 4);
            xv[d] = half == 0 ? xv[d] * cs.x - part * cs.y : xv[d] * cs.x + part * cs.y;
          });
        } else {
          // pair index j = half * D/4 + d/2: the row axis in half 0, the
          // column axis in half 1, frequency d/2 in both
          static_for<HD / 2>([&](auto i_c) {
            constexpr int d = 2 * decltype(i_c)::value;
            const float2 cs = cos_sin(std::integral_constant<int, d / 2>{}, half != 0);
            const float a = xv[d], b = xv[d + 1];
            xv[d] = a * cs.x - b * cs.y;
            xv[d + 1] = b * cs.x + a * cs.y;
          });
        }
      }
    };
    if (qpre.weight != nullptr || qpre.pos != nullptr) {
      int2 pr = make_int2(0, 0);
      if (qpre.pos != nullptr && qrow < len)
        pr = *reinterpret_cast<const int2*>(qpre.pos + 2 * (start + qrow));
      prep_row(qv, qpre.weight, pr);
    }
    float m = -INFINITY, l = 0.f;
    // Keys visited: the segment, or with CAUSAL those up to the unit's last row.
    const int kv_end = CAUSAL ? min(len, qt * kBM + kBM) : len;

    for (int kv0 = 0; kv0 < kv_end; kv0 += kBN) {
      __syncthreads();  // previous tile fully consumed
      for (int c = lane; c < kBN * (D / 4); c += kThreads) {
        const int key = c / (D / 4);
        const int dc = c - key * (D / 4);
        float4 kx = make_float4(0.f, 0.f, 0.f, 0.f), vx = kx;
        if (kv0 + key < kv_end) {
          const size_t tok = size_t(start + kv0 + key);
          kx = *reinterpret_cast<const float4*>(k + tok * ts.k + size_t(h) * D + dc * 4);
          vx = *reinterpret_cast<const float4*>(v + tok * ts.v + size_t(h) * D + dc * 4);
        }
        *reinterpret_cast<float4*>(ks + key * ROW + dc * 4) = kx;
        *reinterpret_cast<float4*>(vs + key * ROW + dc * 4) = vx;
      }
      __syncthreads();
      const int nk = kv_end - kv0 < kBN ? kv_end - kv0 : kBN;
      if (qpre.fuse_k && r < nk) {
        // fuse_k: key row r of the tile, normalised and rotated in place by
        // its lane pair (both lanes of a pair take this branch together)
        float* const kr = ks + r * ROW + half * HD;
        float kv[HD];
#pragma unroll
        for (int d = 0; d < HD; ++d) kv[d] = kr[d];
        int2 pr = make_int2(0, 0);
        if (qpre.pos != nullptr) pr = *reinterpret_cast<const int2*>(qpre.pos + 2 * (start + kv0 + r));
        prep_row(kv, qpre.k_weight, pr);
#pragma unroll
        for (int d = 0; d < HD; ++d) kr[d] = kv[d];
      }
      if (qpre.fuse_k) __syncthreads();
      for (int j = 0; j < nk; ++j) {
        const float* kr = ks + j * ROW + half * HD;
        float part = 0.f;
#pragma unroll
        for (int d = 0; d < HD; ++d) part = fmaf(qv[d], kr[d], part);
        const float dot = part + __shfl_xor(part, 32);
        // Causal: keys after this row get weight zero (key 0 always comes
        // first, so m is finite before any such key).
        const float sc = CAUSAL && kv0 + j > qrow ? -INFINITY : dot * scale;
        const float m_new = fmaxf(m, sc);
        const float alpha = expf(m - m_new);
        const float p = expf(sc - m_new);
        m = m_new;
        l = l * alpha + p;
        const float* vr = vs + j * ROW + half * HD;
#pragma unroll
        for (int d = 0; d < HD; ++d) acc[d] = fmaf(p, vr[d], acc[d] * alpha);
      }
    }

    if (qrow < len) {
      // Log-sum-exp of the row's scores (natural log): sum_b e^score = e^m * l.
      if (lse != nullptr && half == 0) lse[size_t(start + qrow) * H + h] = m + logf(l);
      const float inv = 1.f / l;
      float* op = out + size_t(start + qrow) * ts.o + size_t(h) * D + half * HD;
#pragma unroll
      for (int d = 0; d < HD; d += 4)
        *reinterpret_cast<float4*>(op + d) =
            make_float4(acc[d] * inv, acc[d + 1] * inv, acc[d + 2] * inv, acc[d + 3] * inv);
    }
  }
}

template <int D>
hipError_t launch_d(const void* q, const void* k, const void* v, const Schedule& sch, int H,
                    float scale, bool causal, const QPrepass* qp, void* out, float* lse,
                    TokenStrides ts, hipStream_t stream, hipEvent_t e0, hipEvent_t e1) {
  QPrepass qpre{};
  if (qp != nullptr) qpre = *qp;
  const int64_t items = sch.items != nullptr
                            ? sch.cap
                            : int64_t(sch.batch) * ((sch.seq_len + kBM - 1) / kBM);
  const int64_t units = items * int64_t(H);
  if (units <= 0) return hipSuccess;
  const int64_t grid = units < kMaxAttnGrid ? units : kMaxAttnGrid;
  auto kern = causal ? attn_f32_kernel<D, true> : attn_f32_kernel<D, false>;
  hipExtLaunchKernelGGL(kern, dim3(unsigned(grid)), dim3(kThreads), 0, stream, e0, e1, 0,
                     static_cast<const float*>(q), static_cast<const float*>(k),
                     static_cast<const float*>(v), sch.cu, sch.items, sch.meta, sch.batch,
                     sch.seq_len, H, scale, static_cast<float*>(out), lse, ts, qpre);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_f32(const void* q, const void* k, const void* v, const Schedule& sch,
                           int H, int D, float scale, bool causal, const QPrepass* qp, void* out,
                           float* lse, TokenStrides ts, hipStream_t stream, hipEvent_t e0,
                           hipEvent_t e1) {
  switch (D) {
    case 32: return launch_d<32>(q, k, v, sch, H, scale, causal, qp, out, lse, ts, stream, e0, e1);
    case 64: return launch_d<64>(q, k, v, sch, H, scale, causal, qp, out, lse, ts, stream, e0, e1);
    case 80: return launch_d<80>(q, k, v, sch, H, scale, causal, qp, out, lse, ts, stream, e0, e1);
    case 96: return launch_d<96>(q, k, v, sch, H, scale, causal, qp, out, lse, ts, stream, e0, e1);
    case 128: return launch_d<128>(q, k, v, sch, H, scale, causal, qp, out, lse, ts, stream, e0, e1);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace vit
