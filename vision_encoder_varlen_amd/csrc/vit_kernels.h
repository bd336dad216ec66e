// Internal launch interface between the C ABI (vit_abi.hip) and the kernels.
// Not installed; the public interface is include/vit.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace vit {

// Elements between consecutive tokens of each tensor ([T, H, D] contiguous:
// H * D; a view of a packed [T, 3, H, D] projection: 3 * H * D).  Rows of one
// token's heads stay contiguous (head h at offset h * D).
struct TokenStrides {
  int q, k, v, o;
};

// Calls f(std::integral_constant<int, I>{}) for I = 0 .. N-1: a loop whose
// index is a compile-time constant in the body (array indices stay constant,
// so nothing indexed by it is placed in scratch memory).
template <class F, int... I>
__host__ __device__ __attribute__((always_inline)) inline void static_for_impl(
    F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__host__ __device__ __attribute__((always_inline)) inline void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Pre-pass applied by the attention kernels themselves: to each query row as
// they load it (pos == null and weight == null: none), and with fuse_k also to
// each key row of every K tile (k_weight, same pos and rotary).  The rotation
// angle of pair index j for coordinate c is 2*pi * c * rev[j] with rev[j] =
// inv_freq[j] / (2*pi) held as an unevaluated sum rev_hi[j] + rev_lo[j], so
// the angle can be reduced to a fraction of a turn exactly before the hardware
// sine and cosine.
constexpr int kMaxQFreqs = 32;  // D/4 for D <= 128
struct QPrepass {
  const int32_t* pos;    // int32 [T, 2] (row, col), or null: no rotary
  const float* weight;   // fp32 [D] RMSNorm weight of q, or null: no norm
  float eps;
  int rope_mode;         // 0: rotate-half pairs (m, m + D/2); 1: pairs (2j, 2j + 1)
  float rev_hi[kMaxQFreqs];
  float rev_lo[kMaxQFreqs];
  const float* k_weight; // fp32 [D] RMSNorm weight of k (fuse_k), or null: no norm
  int fuse_k;            // 1: k's rows are normalised and rotated in the kernel too
};

// Where the attention kernels take their (segment, q-tile) items from: a
// device work-list (items, meta and cu_seqlens), or, with items == null, a
// uniform batch of `batch` segments of `seq_len` tokens each, segment i
// starting at token i * seq_len (cu_seqlens = arange(0, (batch+1)*seq_len,
// seq_len), never stored), taken in index order.
struct Schedule {
  const int32_t* cu;
  const int32_t* items;  // int32 [cap, 4]: (segment, q-tile, first token, length)
  const int32_t* meta;
  int64_t cap;  // list capacity (work-list form)
  int batch;    // uniform form
  int seq_len;
};

// Every launch_* takes ev_start / ev_stop: both null, or both timing events
// that are recorded at its kernel's dispatch start and end (hipExtLaunchKernel).

// Query rows per (segment, q-tile) work item.
// bf16 MFMA kernel: 32 rows per wave, 8 waves at head dim 80, else 4.
constexpr int bf16_block_m_const(int head_dim) { return head_dim == 80 ? 256 : 128; }
constexpr int kBlockMF32 = 32;  // 1 wave, lane pairs share a row, fp32 kernel

// Work-list builder limits: one workgroup sorts every segment in LDS.
constexpr int kWorklistMaxSeqs = 8192;
// Work items are (segment, q-tile, first token, length), four int32 each.
constexpr int kWorklistItemInts = 4;

// Largest span of one segment's rows in a k or v tensor (bytes) that the
// bf16 attention kernel addresses with 32-bit buffer offsets, counted with the
// key padding of its last tile (up to kMaxKeyTile rows).  Segments that do not
// fit are skipped by the kernel; the C ABI rejects max_seqlen values that
// allow them.
constexpr int64_t kMaxSegmentBytes = int64_t(1) << 30;
constexpr int kMaxKeyTile = 64;
inline __host__ __device__ bool segment_fits(int64_t len, int64_t token_stride) {
  return (len + kMaxKeyTile) * token_stride * 2 <= kMaxSegmentBytes;
}

// Upper bound on attention workgroups per launch; larger work loops inside.
constexpr int64_t kMaxAttnGrid = int64_t(1) << 22;
// The bf16 kernel's bound: four workgroups per resident slot (2 per CU x 256
// CUs).  The dispatcher still balances units across slots, and many short
// units share one workgroup's set-up (copy offsets, LDS tables): 12% faster
// on 2048 segments of 64 tokens, unchanged on the long-segment batches.
constexpr int64_t kMaxAttnGridBf16 = 2048;
// The builder marks this many entries after the last item (or all of the
// list, if shorter) with segment -1.  A bf16 attention workgroup reads items
// b/H, (b + grid)/H, ... (grid <= kMaxAttnGridBf16) and stops at the first
// marked one, which lies within grid/H entries of the count, so it never needs
// the count itself.
constexpr int64_t kWorklistSentinelSpan = kMaxAttnGridBf16;

inline bool attn_head_dim_supported(int D) {
  return D == 32 || D == 64 || D == 80 || D == 96 || D == 128;
}

// A work-list build to run in the same launch as the pre-pass (cu == null:
// none).  npad is filled in by launch_prepass.
struct WorklistJob {
  const int32_t* cu;
  int N;
  int npad;
  int max_seqlen;
  int block_m;
  int32_t* items;
  long long cap;
  int32_t* meta;
};
// Largest work-list LDS (npad * 12 bytes) built inside the pre-pass launch;
// larger lists get a launch of their own.
constexpr size_t kFusedWorklistMaxLds = 24 * 1024;

// Rows the pre-pass reads (q_src, k_src) and writes (q, k), with their token
// strides in elements (0 = H * D).  Sources equal to the outputs, with the
// same strides, are the in-place form; q_src and q are both null when only k
// is processed.
struct PrepassIO {
  const void* q_src;
  const void* k_src;
  void* q;
  void* k;
  int q_src_stride;
  int k_src_stride;
  int q_stride;
  int k_stride;
};

// Pre-pass: inv_freq_host holds the D/4 rotary inverse frequencies in double
// (may be null when pos is null).  dtype: 0 = fp32, 1 = bf16.  With a job,
// the work-list is built by one more workgroup of the same launch (the two
// are independent).
hipError_t launch_prepass(const PrepassIO& io, int64_t T, int H, int D, int dtype,
                          const int32_t* pos, const double* inv_freq_host,
                          const float* wq, const float* wk, float eps, hipStream_t stream,
                          hipEvent_t ev_start, hipEvent_t ev_stop, const WorklistJob* job,
                          int rope_mode);

hipError_t launch_worklist(const int32_t* cu, int N, int max_seqlen, int block_m,
                           int32_t* items, int64_t cap, int32_t* meta, hipStream_t stream,
                           hipEvent_t ev_start, hipEvent_t ev_stop);

// causal: query row a of a segment sees keys 0..a of that segment only.
// qp: optional Q-side pre-pass (null: q is used as stored).
hipError_t launch_attn_bf16(const void* q, const void* k, const void* v, const Schedule& sch,
                            int H, int D, float scale, bool causal, const QPrepass* qp, void* out,
                            float* lse, TokenStrides ts, hipStream_t stream, hipEvent_t ev_start,
                            hipEvent_t ev_stop);
// The same for calls with part of the pre-pass inside the kernel (qp not
// null, with pos, a q weight or fuse_k): the kernels of attn_bf16_fused.hip.
hipError_t launch_attn_bf16_fused(const void* q, const void* k, const void* v, const Schedule& sch,
                                  int H, int D, float scale, bool causal, const QPrepass* qp,
                                  void* out, float* lse, TokenStrides ts, hipStream_t stream,
                                  hipEvent_t ev_start, hipEvent_t ev_stop);

hipError_t launch_attn_f32(const void* q, const void* k, const void* v, const Schedule& sch,
                           int H, int D, float scale, bool causal, const QPrepass* qp, void* out,
                           float* lse, TokenStrides ts, hipStream_t stream, hipEvent_t ev_start,
                           hipEvent_t ev_stop);

// Attention launches: lse (fp32 [T, H], may be null) receives each row's
// log-sum-exp of scores, natural log.

}  // namespace vit
