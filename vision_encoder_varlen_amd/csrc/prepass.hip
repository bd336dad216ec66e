// Fused Q/K RMSNorm + 2D rotary embedding, fp32 arithmetic, in place or from
// separate source rows into the output rows.
//
// Norm: vLLM page vllm.models.dots3_note.nvidia.vision_attention, _RMSNorm
// (mean of squares over the head dim, fp32 reduce, rsqrt, times a [D] weight
// shared by all heads).  Rotary: VisionRotaryEmbedding on the same page, with
// the row index looking up the first D/4 frequencies and the column index the
// next D/4, applied rotate-half to pairs (m, m + D/2) -- the native rotary
// branch of MultimodalEncoderAttention.forward on the tokenspeed page
// mm_encoder_attention.py widens a half-width cosine the same way.  Order: norm,
// then rotary (_qkv_with_rope).  The complex form (position_embedding_mode
// "complex_rope" on the tokenspeed page) turns the same angles on the pairs
// (2j, 2j + 1) instead.
//
// Memory-bound.  A workgroup takes a group of tokens:
//  1. cos/sin of the token group's D/2 angles go to LDS, so each angle is
//     evaluated once per token rather than once per head and tensor (accurate
//     sincosf; the inverse frequencies arrive precomputed in the kernel
//     arguments);
//  2. each (token, head) row is handled by G consecutive lanes of a wave; a
//     lane owns E consecutive dims m..m+E-1 of the first half and their rotary
//     partners m+D/2.., so the rotation is lane-local and only the sum of
//     squares crosses lanes (an xor shuffle when G is a power of two).  E = 8
//     for bf16 rows (16-byte accesses; a D = 80 row takes 5 lanes, so a wave
//     holds 12 rows), else 4.  Every row is read and written exactly once
//     (the source row, then the output row; the same row in place).  A
//     lane issues the four loads of its row (q and k, both halves) before any
//     arithmetic, and token groups are small (about two rows per lane), so
//     many workgroups keep enough loads in flight to approach HBM bandwidth.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "vit_kernels.h"
#include "worklist_build.h"

namespace vit {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxD = 256;

// Inverse frequencies as unevaluated sums hi + lo of two floats (about 48
// significant bits), so the angle pos * inv_freq can be formed to fp32
// accuracy at any position.
struct Freqs {
  float hi[kMaxD / 4];
  float lo[kMaxD / 4];
};

typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned short u16;

__device__ __forceinline__ float bf16_to_f32(unsigned int bits16) {
  return __uint_as_float(bits16 << 16);
}

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// E consecutive elements: one 8- or 16-byte load kept as raw bits, unpacked
// to fp32 only where the values are used, so the loads of a row are all in
// flight before the first wait.
template <int E>
__device__ __forceinline__ u32x4_t loadRaw(const float* p) {
  static_assert(E == 4, "fp32 rows are handled 4 elements per access");
  return *reinterpret_cast<const u32x4_t*>(p);
}
template <int E>
__device__ __forceinline__ void unpackE(const float*, const u32x4_t& v, float x[E]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = __uint_as_float(v[i]);
}
template <int E>
__device__ __forceinline__ void storeE(float* p, const float x[E]) {
  static_assert(E == 4, "fp32 rows are handled 4 elements per access");
  *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
}
template <int E>
__device__ __forceinline__ u32x4_t loadRaw(const u16* p) {
  if constexpr (E == 8) return *reinterpret_cast<const u32x4_t*>(p);
  const u32x2_t v = *reinterpret_cast<const u32x2_t*>(p);
  return u32x4_t{v.x, v.y, 0u, 0u};
}
template <int E>
__device__ __forceinline__ void unpackE(const u16*, const u32x4_t& v, float x[E]) {
#pragma unroll
  for (int i = 0; i < E / 2; ++i) {
    x[2 * i] = bf16_to_f32(v[i] & 0xffffu);
    x[2 * i + 1] = bf16_to_f32(v[i] >> 16);
  }
}
// The norm weights of a lane's E dims (16-byte aligned fp32).
template <int E>
__device__ __forceinline__ void loadWeights(const float* p, float x[E]) {
#pragma unroll
  for (int i = 0; i < E / 4; ++i) {
    const float4 v = *reinterpret_cast<const float4*>(p + 4 * i);
    x[4 * i] = v.x; x[4 * i + 1] = v.y; x[4 * i + 2] = v.z; x[4 * i + 3] = v.w;
  }
}
template <int E>
__device__ __forceinline__ void storeE(u16* p, const float x[E]) {
  __bf16 w[E];
#pragma unroll
  for (int e = 0; e < E; ++e) w[e] = (__bf16)x[e];  // round to nearest even
  if constexpr (E == 8) *reinterpret_cast<u32x4_t*>(p) = __builtin_bit_cast(u32x4_t, w);
  else *reinterpret_cast<u32x2_t*>(p) = __builtin_bit_cast(u32x2_t, w);
}

// Sum of v over the G consecutive lanes [base, base + G) of a row.
__device__ __forceinline__ float row_sum(float v, int G, int base) {
  if ((G & (G - 1)) == 0) {
    for (int off = G >> 1; off > 0; off >>= 1) v += __shfl_xor(v, off);
    return v;
  }
  float t = 0.f;
  for (int j = 0; j < G; ++j) t += __shfl(v, base + j);
  return t;
}

// Each lane loads all of its row elements before it stores any, and no
// other lane touches that row, so a source row may be its own output row.
template <typename T, int E>
__global__ __launch_bounds__(kThreads) void prepass_kernel(
    const T* qi, const T* ki, T* q, T* k, long long T_tok, int H, int D, int G, int tok_per_grp,
    const int32_t* __restrict__ pos, Freqs freqs, const float* __restrict__ wq,
    const float* __restrict__ wk, float eps, WorklistJob job, int qsi, int ksi, int qs, int ks,
    int rope_mode) {
  extern __shared__ float2 cs[];  // [tok_per_grp][D/2] (cos, sin)
  __shared__ int s_wave[kThreads / 64];
  // With a work-list job workgroup 0 (dispatched first) builds the list,
  // independent of the pre-pass, and the others share the token groups.
  const int npre = job.cu != nullptr ? int(gridDim.x) - 1 : int(gridDim.x);
  const int pblock = job.cu != nullptr ? int(blockIdx.x) - 1 : int(blockIdx.x);
  if (pblock < 0) {
    unsigned long long* keys = reinterpret_cast<unsigned long long*>(cs);
    wl::build_worklist<kThreads>(job.cu, job.N, job.npad, job.max_seqlen, job.block_m, job.items,
                                 job.cap, job.meta, keys, reinterpret_cast<int*>(keys + job.npad),
                                 s_wave);
    return;
  }
  const int tid = threadIdx.x;
  const int half_d = D / 2;
  const int quarter_d = D / 4;
  const bool rope = pos != nullptr;
  const bool norm = wk != nullptr;    // wq too, when q is given
  const bool has_q = q != nullptr;    // null: k only (q is rotated elsewhere)
  const float inv_d = 1.f / float(D);

  // A row takes G consecutive lanes of a wave; a wave holds 64 / G rows.
  const int lane = tid & 63;
  const int rows_per_wave = 64 / G;
  const int rw = lane / G;
  const int lane_g = lane - rw * G;       // lane inside the row
  const int m0 = lane_g * E;              // first dim of this lane (first half)
  const bool lane_active = rw < rows_per_wave;
  const int rows_per_pass = (kThreads / 64) * rows_per_wave;
  const int row_in_pass = (tid >> 6) * rows_per_wave + rw;
  // Norm weights of this lane's dims, the same for every row.
  float wa[2][E] = {}, wb[2][E] = {};
  if (norm && lane_active) {
    if (has_q) {
      loadWeights<E>(wq + m0, wa[0]);
      loadWeights<E>(wq + m0 + half_d, wb[0]);
    }
    loadWeights<E>(wk + m0, wa[1]);
    loadWeights<E>(wk + m0 + half_d, wb[1]);
  }

  // One pass of rows: the loads (issued before any arithmetic, both tensors,
  // so each lane keeps four independent loads in flight), then norm, rotary
  // and stores.
  struct Rows {
    u32x4_t ra[2], rb[2];  // raw loads: first and second half of q's and k's row
    size_t qbase, kbase;
    int tl;
    bool row_ok;
  };
  // A lane without a row reads the group's row 0 and discards it, so no
  // per-lane branch surrounds the loads.
  auto load_rows = [&](long long t0, int ntok, int r0) {
    Rows rw_;
    const int row = r0 + row_in_pass;  // (token_local, head) row inside the group
    rw_.row_ok = row < ntok * H && lane_active;
    const int tl = row / H;
    const int h = row - tl * H;
    rw_.tl = tl;
    rw_.qbase = size_t(t0 + tl) * qs + size_t(h) * D;
    rw_.kbase = size_t(t0 + tl) * ks + size_t(h) * D;
    const int ltl = rw_.row_ok ? tl : 0, lh = rw_.row_ok ? h : 0;
    const size_t qibase = size_t(t0 + ltl) * qsi + size_t(lh) * D;
    const size_t kibase = size_t(t0 + ltl) * ksi + size_t(lh) * D;
    rw_.ra[0] = rw_.rb[0] = u32x4_t{0u, 0u, 0u, 0u};
    if (has_q) {
      rw_.ra[0] = loadRaw<E>(qi + qibase + m0);
      rw_.rb[0] = loadRaw<E>(qi + qibase + m0 + half_d);
    }
    rw_.ra[1] = loadRaw<E>(ki + kibase + m0);
    rw_.rb[1] = loadRaw<E>(ki + kibase + m0 + half_d);
    return rw_;
  };
  auto finish_rows = [&](Rows& rw_) {
    float a[2][E], b[2][E];
#pragma unroll
    for (int which = 0; which < 2; ++which) {
      unpackE<E>(qi, rw_.ra[which], a[which]);
      unpackE<E>(qi, rw_.rb[which], b[which]);
    }
    const bool row_ok = rw_.row_ok;
    const int tl = rw_.tl;
    const size_t qbase = rw_.qbase, kbase = rw_.kbase;
    if (norm) {
      float ss[2];
#pragma unroll
      for (int which = 0; which < 2; ++which) {
        ss[which] = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e)
          ss[which] = fmaf(a[which][e], a[which][e], fmaf(b[which][e], b[which][e], ss[which]));
        ss[which] = row_sum(ss[which], G, rw * G);
      }
#pragma unroll
      for (int which = 0; which < 2; ++which) {
        const float rinv = rsqrtf(ss[which] * inv_d + eps);
#pragma unroll
        for (int e = 0; e < E; ++e) {
          a[which][e] = a[which][e] * rinv * wa[which][e];
          b[which][e] = b[which][e] * rinv * wb[which][e];
        }
      }
    }
    if (rope && row_ok && rope_mode == 0) {
      // Rotate-half: element m of the first half pairs with m + D/2 and
      // turns by angle m.
      const float2* c = cs + tl * half_d + m0;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float2 cse = c[e];
#pragma unroll
        for (int which = 0; which < 2; ++which) {
          const float ya = a[which][e] * cse.x - b[which][e] * cse.y;
          const float yb = b[which][e] * cse.x + a[which][e] * cse.y;
          a[which][e] = ya;
          b[which][e] = yb;
        }
      }
    } else if (rope && row_ok) {
      // Complex form: elements (2j, 2j+1) are one complex number turned by
      // angle j.  This lane's first-half dims hold pairs m0/2 .., its
      // second-half dims pairs D/4 + m0/2 ..
      const float2* ca = cs + tl * half_d + m0 / 2;
      const float2* cb = ca + quarter_d;
#pragma unroll
      for (int i = 0; i < E / 2; ++i) {
        const float2 c1 = ca[i], c2 = cb[i];
#pragma unroll
        for (int which = 0; which < 2; ++which) {
          const float a0 = a[which][2 * i], a1 = a[which][2 * i + 1];
          a[which][2 * i] = a0 * c1.x - a1 * c1.y;
          a[which][2 * i + 1] = a1 * c1.x + a0 * c1.y;
          const float b0 = b[which][2 * i], b1 = b[which][2 * i + 1];
          b[which][2 * i] = b0 * c2.x - b1 * c2.y;
          b[which][2 * i + 1] = b1 * c2.x + b0 * c2.y;
        }
      }
    }
    if (row_ok) {
      if (has_q) {
        storeE<E>(q + qbase + m0, a[0]);
        storeE<E>(q + qbase + m0 + half_d, b[0]);
      }
      storeE<E>(k + kbase + m0, a[1]);
      storeE<E>(k + kbase + m0 + half_d, b[1]);
    }
  };

  for (long long t0 = (long long)pblock * tok_per_grp; t0 < T_tok;
       t0 += (long long)npre * tok_per_grp) {
    const int ntok = T_tok - t0 < tok_per_grp ? int(T_tok - t0) : tok_per_grp;
    // The first pass of rows is loaded before the cos/sin table's inputs, so
    // the two fetches overlap: the table waits once for both (loads complete
    // in order), instead of its inputs' latency and then the rows' one after
    // the other.
    auto table_entry = [&](int i, int coord_i, float f_hi, float f_lo) {
      const float coord = float(coord_i);
      // angle = a_hi + a_lo exactly up to the rounding of a_lo: fmaf recovers
      // the rounding error of coord * hi.
      const float a_hi = coord * f_hi;
      const float a_lo = fmaf(coord, f_hi, -a_hi) + coord * f_lo;
      float sn, cn;
      sincosf(a_hi, &sn, &cn);
      // first-order correction for a_lo (|a_lo| <= 2^-23 |a_hi|; the neglected
      // second-order term is below 2^-46 |a_hi|^2)
      cs[i] = make_float2(fmaf(-sn, a_lo, cn), fmaf(cn, a_lo, sn));
    };
    // entry i: token i / (D/2), pair m = i mod (D/2); the row coordinate for
    // m < D/4, the column for the rest, with frequency m mod D/4
    auto entry_coord = [&](int i) {
      const int tl = i / half_d;
      const int m = i - tl * half_d;
      return pos[2 * (t0 + tl) + (m < quarter_d ? 0 : 1)];
    };
    auto entry_freq = [&](int i) {
      const int m = i % half_d;
      return m < quarter_d ? m : m - quarter_d;
    };
    Rows first = load_rows(t0, ntok, 0);
    const bool own_entry = rope && tid < ntok * half_d;
    int c0 = 0;
    float h0 = 0.f, l0 = 0.f;
    if (rope) {  // uniform; a thread without an entry reads entry 0's inputs
      const int ei = own_entry ? tid : 0;
      c0 = entry_coord(ei);
      h0 = freqs.hi[entry_freq(ei)];
      l0 = freqs.lo[entry_freq(ei)];
    }
    if (rope) {
      if (own_entry) table_entry(tid, c0, h0, l0);
      for (int i = tid + kThreads; i < ntok * half_d; i += kThreads) {
        const int j = entry_freq(i);
        table_entry(i, entry_coord(i), freqs.hi[j], freqs.lo[j]);
      }
      __syncthreads();
    }
    finish_rows(first);
    for (int r0 = rows_per_pass; r0 < ntok * H; r0 += rows_per_pass) {
      Rows cur = load_rows(t0, ntok, r0);
      finish_rows(cur);
    }
    if (rope) __syncthreads();  // cs is rewritten by the next token group
  }
}

}  // namespace

hipError_t launch_prepass(const PrepassIO& io, int64_t T, int H, int D, int dtype,
                          const int32_t* pos, const double* inv_freq_host, const float* wq,
                          const float* wk, float eps, hipStream_t stream, hipEvent_t e0,
                          hipEvent_t e1, const WorklistJob* job, int rope_mode) {
  const int qs = io.q_stride > 0 ? io.q_stride : H * D;
  const int ks = io.k_stride > 0 ? io.k_stride : H * D;
  const int qsi = io.q_src_stride > 0 ? io.q_src_stride : H * D;
  const int ksi = io.k_src_stride > 0 ? io.k_src_stride : H * D;
  WorklistJob jb{};
  if (job != nullptr) jb = *job;
  // Out of place, rows are copied even with neither norm nor rotary.
  const bool in_place = io.q_src == io.q && io.k_src == io.k && qsi == qs && ksi == ks;
  const bool prepass_work = T > 0 && (pos != nullptr || wk != nullptr || !in_place);
  if (!prepass_work) {
    if (jb.cu == nullptr) return hipSuccess;
    return launch_worklist(jb.cu, jb.N, jb.max_seqlen, jb.block_m, jb.items, jb.cap, jb.meta,
                           stream, e0, e1);
  }
  // Elements per lane per half row: 8 (one 16-byte access) for bf16 rows
  // whose half is a multiple of 8, else 4.  G lanes cover a row.
  const int E = (dtype == 1 && (D / 2) % 8 == 0) ? 8 : 4;
  const int G = (D / 2) / E;
  const int rows_per_pass = (kThreads / 64) * (64 / G);
  // Two passes of rows per token group (about two rows per lane): many
  // small workgroups keep the most loads in flight, and the cos/sin table is
  // still shared by all heads.  Large batches take four passes when that
  // still leaves at least 2048 workgroups (8 per CU): fewer tables and
  // barriers per row, 6-14% faster on the 28.7k- and 131k-token batches,
  // unchanged on the small ones.
  int passes = 2;
  if (H > 0 && (4 * rows_per_pass) / H > 0 &&
      (T + (4 * rows_per_pass) / H - 1) / ((4 * rows_per_pass) / H) >= 2048)
    passes = 4;
  int tok_per_grp = (passes * rows_per_pass) / H;
  if (tok_per_grp < 1) tok_per_grp = 1;
  const int max_tok_lds = 32768 / (D / 2 * int(sizeof(float) * 2));
  if (tok_per_grp > max_tok_lds) tok_per_grp = max_tok_lds;
  Freqs fr{};
  if (pos != nullptr) {
    for (int j = 0; j < D / 4; ++j) {
      fr.hi[j] = float(inv_freq_host[j]);
      fr.lo[j] = float(inv_freq_host[j] - double(fr.hi[j]));
    }
  }
  const long long groups = (T + tok_per_grp - 1) / tok_per_grp;
  long long grid = groups < 65536 ? groups : 65536;
  size_t lds = pos != nullptr ? size_t(tok_per_grp) * (D / 2) * sizeof(float) * 2 : 0;
  if (jb.cu != nullptr) {
    // One more workgroup builds the work-list in the same launch.
    jb.npad = 1;
    while (jb.npad < jb.N) jb.npad <<= 1;
    const size_t wl_lds = size_t(jb.npad) * (sizeof(unsigned long long) + sizeof(int));
    if (wl_lds > kFusedWorklistMaxLds) {
      // Too large to share the pre-pass's LDS budget: two launches.
      const hipError_t e = launch_worklist(jb.cu, jb.N, jb.max_seqlen, jb.block_m, jb.items, jb.cap,
                                           jb.meta, stream, nullptr, nullptr);
      if (e != hipSuccess) return e;
      jb = WorklistJob{};
    } else {
      grid += 1;
      if (wl_lds > lds) lds = wl_lds;
    }
  }
  auto launch = [&](auto kernel, const auto* qi, const auto* ki, auto* q, auto* k) {
    hipExtLaunchKernelGGL(kernel, dim3(unsigned(grid)), dim3(kThreads), lds, stream, e0, e1, 0, qi,
                          ki, q, k, (long long)T, H, D, G, tok_per_grp, pos, fr, wq, wk, eps, jb,
                          qsi, ksi, qs, ks, rope_mode);
  };
  if (dtype == 1) {
    const u16* qi = static_cast<const u16*>(io.q_src);
    const u16* ki = static_cast<const u16*>(io.k_src);
    u16* q = static_cast<u16*>(io.q);
    u16* k = static_cast<u16*>(io.k);
    if (E == 8) launch(prepass_kernel<u16, 8>, qi, ki, q, k);
    else launch(prepass_kernel<u16, 4>, qi, ki, q, k);
  } else {
    launch(prepass_kernel<float, 4>, static_cast<const float*>(io.q_src),
           static_cast<const float*>(io.k_src), static_cast<float*>(io.q), static_cast<float*>(io.k));
  }
  return hipGetLastError();
}

}  // namespace vit
