// C ABI of libvit.so (declared in include/vit.h): argument validation on the
// host, error reporting, library-owned work-list scratch, kernel launches.
//
// Every argument check runs before the first HIP runtime call, so a rejected
// call enqueues nothing and touches no device state.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <utility>

#include "vit.h"
#include "vit_kernels.h"

namespace {

// Message of the last failed call on this thread: a fixed buffer, so that
// neither success nor failure allocates host memory.
thread_local char g_last_error[512];

// Events that the next kernel-launching call on this thread records at its
// kernel's dispatch start and end (set by vit_time_next_kernel).
struct TimingHook {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};
thread_local TimingHook g_timing;

TimingHook take_timing() {
  const TimingHook t = g_timing;
  g_timing = TimingHook{};
  return t;
}

// A call that launches no kernel still records the hook's events, back to back.
hipError_t record_empty(const TimingHook& t, hipStream_t stream) {
  if (!t.start) return hipSuccess;
  hipError_t e = hipEventRecord(t.start, stream);
  return e == hipSuccess ? hipEventRecord(t.stop, stream) : e;
}

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(VIT_ERR_HIP, "%s failed: %s", what, hipGetErrorString(e));
}

int ok() {
  g_last_error[0] = '\0';
  return VIT_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Work-list scratch owned by the library: one buffer per (device, stream), so
// calls on different streams never share it.  Layout: meta[4] then items of
// four int32 each (16-byte aligned).
// It grows with stream-ordered allocation (hipFreeAsync of the old buffer and
// hipMallocAsync of the new one, both on the caller's stream), so a call never
// waits on the host for work already queued: the old buffer is released only
// after the stream's earlier kernels have read it.
struct Scratch {
  int32_t* buf = nullptr;
  int64_t cap_items = 0;
};
std::mutex g_mu;
std::map<std::pair<int, hipStream_t>, Scratch> g_scratch;

constexpr int64_t kMaxCapacity = int64_t(1) << 30;

int64_t capacity(int num_seqs, int max_seqlen, int block_m) {
  if (num_seqs < 0 || max_seqlen < 0 || block_m <= 0) return -1;
  return int64_t(num_seqs) * ((int64_t(max_seqlen) + block_m - 1) / block_m);
}

int get_scratch(hipStream_t stream, int64_t cap, Scratch** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lock(g_mu);
  Scratch& s = g_scratch[{dev, stream}];
  if (s.cap_items < cap) {
    if (s.buf != nullptr) {
      e = hipFreeAsync(s.buf, stream);
      if (e != hipSuccess) return hip_fail(e, "hipFreeAsync (work-list scratch)");
      s.buf = nullptr;
      s.cap_items = 0;
    }
    int64_t grow = cap < 4096 ? 4096 : cap + cap / 4;
    e = hipMallocAsync(reinterpret_cast<void**>(&s.buf),
                       size_t(4 + vit::kWorklistItemInts * grow) * sizeof(int32_t), stream);
    if (e != hipSuccess) return hip_fail(e, "hipMallocAsync (work-list scratch)");
    s.cap_items = grow;
  }
  *out = &s;
  return VIT_OK;
}

// Work-list scratch of vit_varlen_attn_noalloc, for callers that cannot
// allocate: a fixed device array (meta[4], then kNoAllocMaxItems items of four
// int32; 4 MiB + 16 B), one copy per GPU, held until the process ends.  In host
// code `scratch` names a host-side stand-in, not device memory: host code uses
// only the address hipGetSymbolAddress returns for the current device.
constexpr int64_t kNoAllocMaxItems = int64_t(1) << 18;
static __device__ __align__(256) int32_t scratch[4 + vit::kWorklistItemInts * kNoAllocMaxItems];

constexpr int kNoAllocMaxDevices = 64;
std::mutex g_noalloc_mu;
int32_t* g_noalloc_ptr[kNoAllocMaxDevices];  // device address of `scratch`, per device

// The current device's copy of `scratch`, looked up once per device (on the
// first call made with that device current).
int noalloc_scratch(int32_t** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kNoAllocMaxDevices)
    return fail(VIT_ERR_UNSUPPORTED, "device index %d is beyond the %d this call supports", dev,
                kNoAllocMaxDevices);
  std::lock_guard<std::mutex> lock(g_noalloc_mu);
  if (g_noalloc_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress (no-allocation scratch)");
    if (p == nullptr) return fail(VIT_ERR_HIP, "hipGetSymbolAddress returned a null address");
    g_noalloc_ptr[dev] = static_cast<int32_t*>(p);
  }
  *out = g_noalloc_ptr[dev];
  return VIT_OK;
}

// Checks shared by every attention entry point: the tensors, head count and
// dim, and the scale.
int check_tensor_args(const void* q, const void* k, const void* v, int H, int D, float scale,
                      const void* out) {
  if (!q || !k || !v || !out) return fail(VIT_ERR_INVALID_ARG, "null pointer argument");
  if (H < 1) return fail(VIT_ERR_INVALID_ARG, "num_heads must be >= 1 (got %d)", H);
  if (!vit::attn_head_dim_supported(D))
    return fail(VIT_ERR_UNSUPPORTED, "head_dim %d not supported (supported: 32, 64, 80, 96, 128)", D);
  if (!std::isfinite(scale)) return fail(VIT_ERR_INVALID_ARG, "scale must be finite");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return fail(VIT_ERR_INVALID_ARG, "q, k, v and out must be 16-byte aligned");
  if (out == q || out == k || out == v) return fail(VIT_ERR_INVALID_ARG, "out must not alias q, k or v");
  return VIT_OK;
}

int check_attn_args(const void* q, const void* k, const void* v, const int32_t* cu,
                    int num_seqs, int max_seqlen, int H, int D, float scale, const void* out) {
  if (!cu) return fail(VIT_ERR_INVALID_ARG, "null pointer argument");
  if (num_seqs < 0) return fail(VIT_ERR_INVALID_ARG, "num_seqs must be >= 0 (got %d)", num_seqs);
  if (num_seqs > vit::kWorklistMaxSeqs)
    return fail(VIT_ERR_UNSUPPORTED, "num_seqs %d exceeds the supported maximum %d", num_seqs,
                vit::kWorklistMaxSeqs);
  if (max_seqlen < 0) return fail(VIT_ERR_INVALID_ARG, "max_seqlen must be >= 0 (got %d)", max_seqlen);
  const int rc = check_tensor_args(q, k, v, H, D, scale, out);
  if (rc != VIT_OK) return rc;
  if (!aligned4(cu)) return fail(VIT_ERR_INVALID_ARG, "cu_seqlens must be 4-byte aligned");
  return VIT_OK;
}

int check_flags(int flags) {
  if (flags & ~VIT_ATTN_CAUSAL) return fail(VIT_ERR_INVALID_ARG, "unknown attention flags 0x%x", flags);
  return VIT_OK;
}

int launch_attn(const void* q, const void* k, const void* v, const vit::Schedule& sch, int H,
                int D, float scale, int dtype, int flags, void* out, float* lse,
                const vit::TokenStrides& ts, hipStream_t stream, const TimingHook& t,
                const vit::QPrepass* qp = nullptr) {
  const bool causal = (flags & VIT_ATTN_CAUSAL) != 0;
  const hipError_t e =
      dtype == VIT_BF16
          ? vit::launch_attn_bf16(q, k, v, sch, H, D, scale, causal, qp, out, lse, ts, stream,
                                  t.start, t.stop)
          : vit::launch_attn_f32(q, k, v, sch, H, D, scale, causal, qp, out, lse, ts, stream,
                                 t.start, t.stop);
  return e == hipSuccess ? ok() : hip_fail(e, "attention launch");
}

// Q-side pre-pass parameters for the attention kernels: the same rotary
// frequencies as the pre-pass (theta^(-2j/(D/2)), double), divided by 2*pi
// and split into float hi + lo.
int make_qprepass(int D, const int32_t* pos, float theta, const float* q_weight, float eps,
                  int rope_mode, vit::QPrepass* qp) {
  if (rope_mode != VIT_ROPE_NEOX && rope_mode != VIT_ROPE_COMPLEX)
    return fail(VIT_ERR_INVALID_ARG, "unknown rope_mode %d", rope_mode);
  if (pos != nullptr && (!std::isfinite(theta) || theta <= 0.f))
    return fail(VIT_ERR_INVALID_ARG, "theta must be finite and > 0");
  if (q_weight != nullptr && (!std::isfinite(eps) || eps < 0.f))
    return fail(VIT_ERR_INVALID_ARG, "eps must be finite and >= 0");
  if (pos != nullptr && (reinterpret_cast<uintptr_t>(pos) & 7u) != 0)
    return fail(VIT_ERR_INVALID_ARG, "pos must be 8-byte aligned");
  if (q_weight != nullptr && !aligned16(q_weight))
    return fail(VIT_ERR_INVALID_ARG, "q_weight must be 16-byte aligned");
  *qp = vit::QPrepass{};
  qp->pos = pos;
  qp->weight = q_weight;
  qp->eps = eps;
  qp->rope_mode = rope_mode;
  if (pos != nullptr) {
    const double two_pi = 6.283185307179586476925286766559;
    for (int j = 0; j < D / 4; ++j) {
      const double rev = std::pow(double(theta), -2.0 * j / (D / 2.0)) / two_pi;
      qp->rev_hi[j] = float(rev);
      qp->rev_lo[j] = float(rev - double(qp->rev_hi[j]));
    }
  }
  return VIT_OK;
}

// Token strides (elements) of q, k, v, out from a caller array of n values
// (null: all H * D).  Each must be >= H * D, keep rows 16-byte aligned, and
// stay below 2^26.
int make_strides(const int64_t* st, int n, int H, int D, int dtype, vit::TokenStrides* ts) {
  const int64_t dense = int64_t(H) * D;
  int64_t v[4] = {dense, dense, dense, dense};
  if (st != nullptr)
    for (int i = 0; i < n; ++i) v[i] = st[i];
  const int64_t unit = dtype == VIT_BF16 ? 8 : 4;  // elements per 16 bytes
  for (int i = 0; i < 4; ++i) {
    if (v[i] < dense || v[i] >= (int64_t(1) << 26) || v[i] % unit != 0)
      return fail(VIT_ERR_INVALID_ARG,
                  "token stride %lld must be >= num_heads * head_dim (%lld), < 2^26 and a "
                  "multiple of %lld elements", (long long)v[i], (long long)dense, (long long)unit);
  }
  *ts = vit::TokenStrides{int(v[0]), int(v[1]), int(v[2]), int(v[3])};
  return VIT_OK;
}

int check_lse(const float* lse, const void* q, const void* k, const void* v, const void* out) {
  if (lse == nullptr) return VIT_OK;
  if (!aligned4(lse)) return fail(VIT_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  if (static_cast<const void*>(lse) == q || static_cast<const void*>(lse) == k ||
      static_cast<const void*>(lse) == v || static_cast<const void*>(lse) == out)
    return fail(VIT_ERR_INVALID_ARG, "lse must not alias q, k, v or out");
  return VIT_OK;
}

int block_m_for(int dtype, int D) {
  return dtype == VIT_BF16 ? vit::bf16_block_m_const(D) : vit::kBlockMF32;
}

// noalloc: build the work-list in the fixed device array (`scratch`) instead
// of the per-stream buffer; nothing is allocated.
int attn_common(const void* q, const void* k, const void* v, const int32_t* cu, int num_seqs,
                int max_seqlen, int H, int D, float scale, int flags, void* out, float* lse,
                const int64_t* strides, hipStream_t stream, int dtype, bool noalloc = false) {
  const TimingHook t = take_timing();
  int rc = check_attn_args(q, k, v, cu, num_seqs, max_seqlen, H, D, scale, out);
  if (rc != VIT_OK) return rc;
  rc = check_flags(flags);
  if (rc != VIT_OK) return rc;
  rc = check_lse(lse, q, k, v, out);
  if (rc != VIT_OK) return rc;
  vit::TokenStrides ts{};
  rc = make_strides(strides, 4, H, D, dtype, &ts);
  if (rc != VIT_OK) return rc;
  if (!vit::segment_fits(max_seqlen, ts.k > ts.v ? ts.k : ts.v))
    return fail(VIT_ERR_UNSUPPORTED, "(max_seqlen + %d) * token stride * 2 bytes exceeds %lld",
                vit::kMaxKeyTile, (long long)vit::kMaxSegmentBytes);
  if (num_seqs == 0 || max_seqlen == 0) {
    const hipError_t e = record_empty(t, stream);
    return e == hipSuccess ? ok() : hip_fail(e, "hipEventRecord");
  }
  const int bm = block_m_for(dtype, D);
  const int64_t cap = capacity(num_seqs, max_seqlen, bm);
  if (cap > kMaxCapacity) return fail(VIT_ERR_UNSUPPORTED, "work-list capacity %lld too large", (long long)cap);
  int32_t* buf = nullptr;
  if (noalloc) {
    if (cap > kNoAllocMaxItems)
      return fail(VIT_ERR_UNSUPPORTED,
                  "work-list capacity %lld (num_seqs * ceil(max_seqlen / %d)) exceeds the %lld "
                  "items of the no-allocation scratch", (long long)cap, bm,
                  (long long)kNoAllocMaxItems);
    rc = noalloc_scratch(&buf);
    if (rc != VIT_OK) return rc;
  } else {
    Scratch* s = nullptr;
    rc = get_scratch(stream, cap, &s);
    if (rc != VIT_OK) return rc;
    buf = s->buf;
  }
  int32_t* meta = buf;
  int32_t* items = buf + 4;
  hipError_t e = vit::launch_worklist(cu, num_seqs, max_seqlen, bm, items, cap, meta, stream,
                                      nullptr, nullptr);
  if (e != hipSuccess) return hip_fail(e, "work-list launch");
  return launch_attn(q, k, v, vit::Schedule{cu, items, meta, cap, 0, 0}, H, D, scale, dtype, flags,
                     out, lse, ts, stream, t);
}

int check_prepass_args(void* q, void* k, int64_t total_tokens, int num_heads, int head_dim,
                       int dtype, const int32_t* pos, float theta, const float* q_weight,
                       const float* k_weight, float eps, int rope_mode) {
  if (!k) return fail(VIT_ERR_INVALID_ARG, "null k (q may be null, k may not)");
  if (rope_mode != VIT_ROPE_NEOX && rope_mode != VIT_ROPE_COMPLEX)
    return fail(VIT_ERR_INVALID_ARG, "unknown rope_mode %d", rope_mode);
  if (total_tokens < 0) return fail(VIT_ERR_INVALID_ARG, "total_tokens must be >= 0");
  if (num_heads < 1) return fail(VIT_ERR_INVALID_ARG, "num_heads must be >= 1 (got %d)", num_heads);
  if (head_dim < 8 || head_dim > 256 || head_dim % 8 != 0)
    return fail(VIT_ERR_UNSUPPORTED, "head_dim must be a multiple of 8 in [8, 256] (got %d)", head_dim);
  if (dtype != VIT_F32 && dtype != VIT_BF16) return fail(VIT_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (q == nullptr && q_weight != nullptr)
    return fail(VIT_ERR_INVALID_ARG, "q_weight given without q");
  if (q != nullptr && (q_weight == nullptr) != (k_weight == nullptr))
    return fail(VIT_ERR_INVALID_ARG, "give both q_weight and k_weight or neither");
  if (pos != nullptr && (!std::isfinite(theta) || theta <= 0.f))
    return fail(VIT_ERR_INVALID_ARG, "theta must be finite and > 0");
  if (k_weight != nullptr && (!std::isfinite(eps) || eps < 0.f))
    return fail(VIT_ERR_INVALID_ARG, "eps must be finite and >= 0");
  if (!aligned16(q) || !aligned16(k)) return fail(VIT_ERR_INVALID_ARG, "q and k must be 16-byte aligned");
  if ((q_weight && !aligned16(q_weight)) || (k_weight && !aligned16(k_weight)))
    return fail(VIT_ERR_INVALID_ARG, "norm weights must be 16-byte aligned");
  if (pos && !aligned4(pos)) return fail(VIT_ERR_INVALID_ARG, "pos must be 4-byte aligned");
  if (q == k) return fail(VIT_ERR_INVALID_ARG, "q and k must be distinct buffers");
  return VIT_OK;
}

int check_worklist_args(const int32_t* cu_seqlens, int num_seqs, int max_seqlen, int block_m,
                        int32_t* items, int64_t cap, int32_t* meta) {
  if (!cu_seqlens || !items || !meta) return fail(VIT_ERR_INVALID_ARG, "null pointer argument");
  if (num_seqs < 0 || max_seqlen < 0) return fail(VIT_ERR_INVALID_ARG, "negative size");
  if (num_seqs > vit::kWorklistMaxSeqs)
    return fail(VIT_ERR_UNSUPPORTED, "num_seqs %d exceeds the supported maximum %d", num_seqs,
                vit::kWorklistMaxSeqs);
  if (block_m <= 0) return fail(VIT_ERR_INVALID_ARG, "block_m must be > 0");
  const int64_t need = capacity(num_seqs, max_seqlen, block_m);
  if (need > kMaxCapacity) return fail(VIT_ERR_UNSUPPORTED, "work-list capacity %lld too large", (long long)need);
  if (cap < need)
    return fail(VIT_ERR_INVALID_ARG, "cap %lld below the required capacity %lld", (long long)cap,
                (long long)need);
  if (!aligned4(cu_seqlens) || !aligned4(meta))
    return fail(VIT_ERR_INVALID_ARG, "int32 buffers must be 4-byte aligned");
  if (!aligned16(items)) return fail(VIT_ERR_INVALID_ARG, "items must be 16-byte aligned");
  return VIT_OK;
}

// [first, last) byte range of a [T, H, D] tensor with `stride` elements per
// token.
struct ByteRange {
  uintptr_t first, last;
};
ByteRange rows_range(const void* p, int64_t T, int64_t stride, int H, int D, int elt) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  if (p == nullptr || T == 0) return ByteRange{a, a};
  return ByteRange{a, a + uintptr_t(((T - 1) * stride + int64_t(H) * D) * elt)};
}
bool overlap(ByteRange x, ByteRange y) {
  return x.first < x.last && y.first < y.last && x.first < y.last && y.first < x.last;
}

// The pre-pass from q_src / k_src into q / k.  Each output either is its own
// source with the same stride (in place: a lane reads its row before it
// writes it) or shares no byte with either source; anything else could let
// one lane's stores land on rows another lane has still to read.  job: a
// work-list to build in the same launch, or null.
int prepass_common(const void* q_src, const void* k_src, const int64_t* src_strides, void* q,
                   void* k, int64_t total_tokens, int num_heads, int head_dim, int dtype,
                   const int32_t* pos, float theta, const float* q_weight, const float* k_weight,
                   float eps, int rope_mode, const int64_t* strides, const vit::WorklistJob* job,
                   hipStream_t stream, const TimingHook& t) {
  int rc = check_prepass_args(q, k, total_tokens, num_heads, head_dim, dtype, pos, theta,
                              q_weight, k_weight, eps, rope_mode);
  if (rc != VIT_OK) return rc;
  if (!k_src) return fail(VIT_ERR_INVALID_ARG, "null k_src");
  if ((q_src == nullptr) != (q == nullptr))
    return fail(VIT_ERR_INVALID_ARG, "q_src and q must both be given or both be null");
  if (!aligned16(q_src) || !aligned16(k_src))
    return fail(VIT_ERR_INVALID_ARG, "q_src and k_src must be 16-byte aligned");
  vit::TokenStrides ts{}, tsi{};
  rc = make_strides(strides, 2, num_heads, head_dim, dtype, &ts);
  if (rc != VIT_OK) return rc;
  rc = make_strides(src_strides, 2, num_heads, head_dim, dtype, &tsi);
  if (rc != VIT_OK) return rc;
  const int elt = dtype == VIT_BF16 ? 2 : 4;
  const ByteRange src[2] = {rows_range(q_src, total_tokens, tsi.q, num_heads, head_dim, elt),
                            rows_range(k_src, total_tokens, tsi.k, num_heads, head_dim, elt)};
  const void* outs[2] = {q, k};
  const void* srcs[2] = {q_src, k_src};
  const int out_stride[2] = {ts.q, ts.k};
  const int src_stride[2] = {tsi.q, tsi.k};
  for (int i = 0; i < 2; ++i) {
    if (outs[i] == nullptr) continue;
    if (outs[i] == srcs[i]) {
      if (out_stride[i] != src_stride[i])
        return fail(VIT_ERR_INVALID_ARG, "%s is updated in place but its two strides differ",
                    i == 0 ? "q" : "k");
      // In place, q and k may interleave (views of one packed QKV buffer):
      // their rows are distinct, which the check q != k covers as before.
      continue;
    }
    const ByteRange r = rows_range(outs[i], total_tokens, out_stride[i], num_heads, head_dim, elt);
    if (overlap(r, src[0]) || overlap(r, src[1]))
      return fail(VIT_ERR_INVALID_ARG,
                  "%s overlaps q_src or k_src (an output is either its own source, in place, or "
                  "disjoint from both sources)", i == 0 ? "q" : "k");
  }
  const vit::PrepassIO io{q_src, k_src, q, k, tsi.q, tsi.k, ts.q, ts.k};
  const bool in_place = q_src == q && k_src == k;
  const bool prepass_work =
      total_tokens > 0 && (pos != nullptr || k_weight != nullptr || !in_place);
  if (!prepass_work && job == nullptr) {
    const hipError_t e = record_empty(t, stream);
    return e == hipSuccess ? ok() : hip_fail(e, "hipEventRecord");
  }
  // Rotary inverse frequencies for dim = D/2: theta^(-2j/(D/2)), in double.
  double inv_freq[64];
  const int F = head_dim / 4;
  for (int j = 0; j < F; ++j) inv_freq[j] = std::pow(double(theta), -2.0 * j / (head_dim / 2.0));
  hipError_t e = vit::launch_prepass(io, total_tokens, num_heads, head_dim, dtype, pos, inv_freq,
                                     q_weight, k_weight, eps, stream, t.start, t.stop, job,
                                     rope_mode);
  if (e != hipSuccess) return hip_fail(e, job ? "pre-pass + work-list launch" : "pre-pass launch");
  return ok();
}

}  // namespace

extern "C" {

int vit_qk_norm_rope(void* q, void* k, int64_t total_tokens, int num_heads, int head_dim,
                     int dtype, const int32_t* pos, float theta, const float* q_weight,
                     const float* k_weight, float eps, hipStream_t stream) {
  return vit_qk_norm_rope_strided(q, k, total_tokens, num_heads, head_dim, dtype, pos, theta,
                                  q_weight, k_weight, eps, nullptr, stream);
}

int vit_qk_norm_rope_strided(void* q, void* k, int64_t total_tokens, int num_heads, int head_dim,
                             int dtype, const int32_t* pos, float theta, const float* q_weight,
                             const float* k_weight, float eps, const int64_t* strides,
                             hipStream_t stream) {
  return vit_qk_norm_rope_ex(q, k, total_tokens, num_heads, head_dim, dtype, pos, theta, q_weight,
                             k_weight, eps, VIT_ROPE_NEOX, strides, stream);
}

int vit_qk_norm_rope_ex(void* q, void* k, int64_t total_tokens, int num_heads, int head_dim,
                        int dtype, const int32_t* pos, float theta, const float* q_weight,
                        const float* k_weight, float eps, int rope_mode, const int64_t* strides,
                        hipStream_t stream) {
  const TimingHook t = take_timing();
  return prepass_common(q, k, strides, q, k, total_tokens, num_heads, head_dim, dtype, pos, theta,
                        q_weight, k_weight, eps, rope_mode, strides, nullptr, stream, t);
}

int vit_qk_norm_rope_worklist(void* q, void* k, int64_t total_tokens, int num_heads, int head_dim,
                              int dtype, const int32_t* pos, float theta, const float* q_weight,
                              const float* k_weight, float eps, int rope_mode,
                              const int64_t* strides, const int32_t* cu_seqlens, int num_seqs,
                              int max_seqlen, int block_m, int32_t* items, int64_t cap,
                              int32_t* meta, hipStream_t stream) {
  return vit_qk_norm_rope_into(q, k, strides, q, k, total_tokens, num_heads, head_dim, dtype, pos,
                               theta, q_weight, k_weight, eps, rope_mode, strides, cu_seqlens,
                               num_seqs, max_seqlen, block_m, items, cap, meta, stream);
}

int vit_qk_norm_rope_into(const void* q_src, const void* k_src, const int64_t* src_strides,
                          void* q, void* k, int64_t total_tokens, int num_heads, int head_dim,
                          int dtype, const int32_t* pos, float theta, const float* q_weight,
                          const float* k_weight, float eps, int rope_mode, const int64_t* strides,
                          const int32_t* cu_seqlens, int num_seqs, int max_seqlen, int block_m,
                          int32_t* items, int64_t cap, int32_t* meta, hipStream_t stream) {
  const TimingHook t = take_timing();
  const bool want_list = cu_seqlens != nullptr || items != nullptr || meta != nullptr;
  vit::WorklistJob job{};
  if (want_list) {
    const int rc = check_worklist_args(cu_seqlens, num_seqs, max_seqlen, block_m, items, cap, meta);
    if (rc != VIT_OK) return rc;
    job = vit::WorklistJob{cu_seqlens, num_seqs, 0, max_seqlen, block_m, items, cap, meta};
  }
  return prepass_common(q_src, k_src, src_strides, q, k, total_tokens, num_heads, head_dim, dtype,
                        pos, theta, q_weight, k_weight, eps, rope_mode, strides,
                        want_list ? &job : nullptr, stream, t);
}

int vit_varlen_attn(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                    int num_seqs, int max_seqlen, int num_heads, int head_dim, float scale,
                    void* out, hipStream_t stream) {
  return attn_common(q, k, v, cu_seqlens, num_seqs, max_seqlen, num_heads, head_dim, scale, 0, out,
                     nullptr, nullptr, stream, VIT_BF16);
}

int vit_varlen_attn_f32(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                        int num_seqs, int max_seqlen, int num_heads, int head_dim, float scale,
                        void* out, hipStream_t stream) {
  return attn_common(q, k, v, cu_seqlens, num_seqs, max_seqlen, num_heads, head_dim, scale, 0, out,
                     nullptr, nullptr, stream, VIT_F32);
}

int vit_varlen_attn_lse(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                        int num_seqs, int max_seqlen, int num_heads, int head_dim, float scale,
                        int dtype, void* out, float* lse, hipStream_t stream) {
  if (dtype != VIT_F32 && dtype != VIT_BF16) return fail(VIT_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  return attn_common(q, k, v, cu_seqlens, num_seqs, max_seqlen, num_heads, head_dim, scale, 0, out,
                     lse, nullptr, stream, dtype);
}

int vit_varlen_attn_strided(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                            int num_seqs, int max_seqlen, int num_heads, int head_dim, float scale,
                            int dtype, void* out, float* lse, const int64_t* strides,
                            hipStream_t stream) {
  return vit_varlen_attn_ex(q, k, v, cu_seqlens, num_seqs, max_seqlen, num_heads, head_dim, scale,
                            dtype, 0, out, lse, strides, stream);
}

int vit_varlen_attn_ex(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                       int num_seqs, int max_seqlen, int num_heads, int head_dim, float scale,
                       int dtype, int flags, void* out, float* lse, const int64_t* strides,
                       hipStream_t stream) {
  if (dtype != VIT_F32 && dtype != VIT_BF16) return fail(VIT_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  return attn_common(q, k, v, cu_seqlens, num_seqs, max_seqlen, num_heads, head_dim, scale, flags,
                     out, lse, strides, stream, dtype);
}

int vit_varlen_attn_noalloc(const void* q, const void* k, const void* v,
                            const int32_t* cu_seqlens, int num_seqs, int max_seqlen,
                            int num_heads, int head_dim, float scale, int dtype, int flags,
                            void* out, float* lse, const int64_t* strides, hipStream_t stream) {
  if (dtype != VIT_F32 && dtype != VIT_BF16) return fail(VIT_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  return attn_common(q, k, v, cu_seqlens, num_seqs, max_seqlen, num_heads, head_dim, scale, flags,
                     out, lse, strides, stream, dtype, /*noalloc=*/true);
}

int vit_attn_block_m(int num_heads, int head_dim, int dtype) {
  if (num_heads < 1) return -fail(VIT_ERR_INVALID_ARG, "num_heads must be >= 1");
  if (!vit::attn_head_dim_supported(head_dim))
    return -fail(VIT_ERR_UNSUPPORTED, "head_dim %d not supported", head_dim);
  if (dtype != VIT_F32 && dtype != VIT_BF16) return -fail(VIT_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  ok();
  return block_m_for(dtype, head_dim);
}

int64_t vit_worklist_capacity(int num_seqs, int max_seqlen, int block_m) {
  return capacity(num_seqs, max_seqlen, block_m);
}

int vit_varlen_worklist(const int32_t* cu_seqlens, int num_seqs, int max_seqlen, int block_m,
                        int32_t* items, int64_t cap, int32_t* meta, hipStream_t stream) {
  const TimingHook t = take_timing();
  const int rc = check_worklist_args(cu_seqlens, num_seqs, max_seqlen, block_m, items, cap, meta);
  if (rc != VIT_OK) return rc;
  hipError_t e = vit::launch_worklist(cu_seqlens, num_seqs, max_seqlen, block_m, items, cap, meta,
                                      stream, t.start, t.stop);
  if (e != hipSuccess) return hip_fail(e, "work-list launch");
  return ok();
}

int vit_varlen_attn_planned(const void* q, const void* k, const void* v,
                            const int32_t* cu_seqlens, const int32_t* items, int64_t cap,
                            const int32_t* meta, int num_heads, int head_dim, float scale,
                            int dtype, int flags, void* out, float* lse, const int64_t* strides,
                            hipStream_t stream) {
  const TimingHook t = take_timing();
  if (!items || !meta) return fail(VIT_ERR_INVALID_ARG, "null work-list pointer");
  if (!aligned16(items)) return fail(VIT_ERR_INVALID_ARG, "items must be 16-byte aligned");
  if (dtype != VIT_F32 && dtype != VIT_BF16) return fail(VIT_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  int rc = check_attn_args(q, k, v, cu_seqlens, 0, 0, num_heads, head_dim, scale, out);
  if (rc != VIT_OK) return rc;
  rc = check_flags(flags);
  if (rc != VIT_OK) return rc;
  if (cap < 0 || cap > kMaxCapacity) return fail(VIT_ERR_INVALID_ARG, "bad work-list capacity %lld", (long long)cap);
  rc = check_lse(lse, q, k, v, out);
  if (rc != VIT_OK) return rc;
  vit::TokenStrides ts{};
  rc = make_strides(strides, 4, num_heads, head_dim, dtype, &ts);
  if (rc != VIT_OK) return rc;
  if (cap == 0) {
    const hipError_t e = record_empty(t, stream);
    return e == hipSuccess ? ok() : hip_fail(e, "hipEventRecord");
  }
  return launch_attn(q, k, v, vit::Schedule{cu_seqlens, items, meta, cap, 0, 0}, num_heads,
                     head_dim, scale, dtype, flags, out, lse, ts, stream, t);
}

int vit_varlen_attn_planned_qnorm_rope(
    const void* q, const void* k, const void* v, const int32_t* cu_seqlens, const int32_t* items,
    int64_t cap, const int32_t* meta, int num_heads, int head_dim, float scale, int dtype,
    int flags, const int32_t* pos, float theta, const float* q_weight, float eps, int rope_mode,
    void* out, float* lse, const int64_t* strides, hipStream_t stream) {
  const TimingHook t = take_timing();
  if (!items || !meta) return fail(VIT_ERR_INVALID_ARG, "null work-list pointer");
  if (!aligned16(items)) return fail(VIT_ERR_INVALID_ARG, "items must be 16-byte aligned");
  if (dtype != VIT_F32 && dtype != VIT_BF16) return fail(VIT_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  int rc = check_attn_args(q, k, v, cu_seqlens, 0, 0, num_heads, head_dim, scale, out);
  if (rc != VIT_OK) return rc;
  rc = check_flags(flags);
  if (rc != VIT_OK) return rc;
  if (cap < 0 || cap > kMaxCapacity) return fail(VIT_ERR_INVALID_ARG, "bad work-list capacity %lld", (long long)cap);
  rc = check_lse(lse, q, k, v, out);
  if (rc != VIT_OK) return rc;
  vit::TokenStrides ts{};
  rc = make_strides(strides, 4, num_heads, head_dim, dtype, &ts);
  if (rc != VIT_OK) return rc;
  vit::QPrepass qp{};
  rc = make_qprepass(head_dim, pos, theta, q_weight, eps, rope_mode, &qp);
  if (rc != VIT_OK) return rc;
  if (cap == 0) {
    const hipError_t e = record_empty(t, stream);
    return e == hipSuccess ? ok() : hip_fail(e, "hipEventRecord");
  }
  return launch_attn(q, k, v, vit::Schedule{cu_seqlens, items, meta, cap, 0, 0}, num_heads,
                     head_dim, scale, dtype, flags, out, lse, ts, stream, t, &qp);
}

int vit_varlen_attn_planned_qk_norm_rope(
    const void* q, const void* k, const void* v, const int32_t* cu_seqlens, const int32_t* items,
    int64_t cap, const int32_t* meta, int num_heads, int head_dim, float scale, int dtype,
    int flags, const int32_t* pos, float theta, const float* q_weight, const float* k_weight,
    float eps, int rope_mode, void* out, float* lse, const int64_t* strides, hipStream_t stream) {
  const TimingHook t = take_timing();
  if (!items || !meta) return fail(VIT_ERR_INVALID_ARG, "null work-list pointer");
  if (!aligned16(items)) return fail(VIT_ERR_INVALID_ARG, "items must be 16-byte aligned");
  if (dtype != VIT_F32 && dtype != VIT_BF16) return fail(VIT_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  int rc = check_attn_args(q, k, v, cu_seqlens, 0, 0, num_heads, head_dim, scale, out);
  if (rc != VIT_OK) return rc;
  rc = check_flags(flags);
  if (rc != VIT_OK) return rc;
  if (cap < 0 || cap > kMaxCapacity) return fail(VIT_ERR_INVALID_ARG, "bad work-list capacity %lld", (long long)cap);
  rc = check_lse(lse, q, k, v, out);
  if (rc != VIT_OK) return rc;
  vit::TokenStrides ts{};
  rc = make_strides(strides, 4, num_heads, head_dim, dtype, &ts);
  if (rc != VIT_OK) return rc;
  if ((q_weight == nullptr) != (k_weight == nullptr))
    return fail(VIT_ERR_INVALID_ARG, "q_weight and k_weight must both be given or both be null");
  if (k_weight != nullptr && !aligned16(k_weight))
    return fail(VIT_ERR_INVALID_ARG, "k_weight must be 16-byte aligned");
  vit::QPrepass qp{};
  rc = make_qprepass(head_dim, pos, theta, q_weight, eps, rope_mode, &qp);
  if (rc != VIT_OK) return rc;
  qp.k_weight = k_weight;
  qp.fuse_k = 1;
  if (cap == 0) {
    const hipError_t e = record_empty(t, stream);
    return e == hipSuccess ? ok() : hip_fail(e, "hipEventRecord");
  }
  return launch_attn(q, k, v, vit::Schedule{cu_seqlens, items, meta, cap, 0, 0}, num_heads,
                     head_dim, scale, dtype, flags, out, lse, ts, stream, t, &qp);
}

int vit_dense_batch_attn(const void* q, const void* k, const void* v, int batch, int seq_len,
                         int num_heads, int head_dim, float scale, int dtype, int flags,
                         void* out, float* lse, const int64_t* strides, hipStream_t stream) {
  const TimingHook t = take_timing();
  if (dtype != VIT_F32 && dtype != VIT_BF16) return fail(VIT_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  int rc = check_tensor_args(q, k, v, num_heads, head_dim, scale, out);
  if (rc != VIT_OK) return rc;
  rc = check_flags(flags);
  if (rc != VIT_OK) return rc;
  if (batch < 0 || seq_len < 0)
    return fail(VIT_ERR_INVALID_ARG, "batch and seq_len must be >= 0 (got %d, %d)", batch, seq_len);
  if (int64_t(batch) * seq_len > INT32_MAX)
    return fail(VIT_ERR_UNSUPPORTED, "batch * seq_len must fit in int32");
  rc = check_lse(lse, q, k, v, out);
  if (rc != VIT_OK) return rc;
  vit::TokenStrides ts{};
  rc = make_strides(strides, 4, num_heads, head_dim, dtype, &ts);
  if (rc != VIT_OK) return rc;
  if (!vit::segment_fits(seq_len, ts.k > ts.v ? ts.k : ts.v))
    return fail(VIT_ERR_UNSUPPORTED, "(seq_len + %d) * token stride * 2 bytes exceeds %lld",
                vit::kMaxKeyTile, (long long)vit::kMaxSegmentBytes);
  if (batch == 0 || seq_len == 0) {
    const hipError_t e = record_empty(t, stream);
    return e == hipSuccess ? ok() : hip_fail(e, "hipEventRecord");
  }
  return launch_attn(q, k, v, vit::Schedule{nullptr, nullptr, nullptr, 0, batch, seq_len},
                     num_heads, head_dim, scale, dtype, flags, out, lse, ts, stream, t);
}

int vit_device_error(hipStream_t stream, int32_t* err, int reset) {
  if (!err) return fail(VIT_ERR_INVALID_ARG, "null err pointer");
  *err = 0;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lock(g_mu);
  auto it = g_scratch.find({dev, stream});
  if (it == g_scratch.end() || it->second.buf == nullptr) return ok();
  e = hipMemcpyAsync(err, it->second.buf + 1, sizeof(int32_t), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "reading the work-list error word");
  if (reset) {
    const int32_t zero = 0;
    e = hipMemcpyAsync(it->second.buf + 1, &zero, sizeof(int32_t), hipMemcpyHostToDevice, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_fail(e, "clearing the work-list error word");
  }
  return ok();
}

int vit_time_next_kernel(hipEvent_t start, hipEvent_t stop) {
  if ((start == nullptr) != (stop == nullptr))
    return fail(VIT_ERR_INVALID_ARG, "start and stop must both be events or both be null");
  g_timing = TimingHook{start, stop};
  return ok();
}

const char* vit_last_error(void) { return g_last_error; }

void vit_release(void) {
  std::lock_guard<std::mutex> lock(g_mu);
  for (auto& kv : g_scratch) {
    if (kv.second.buf == nullptr) continue;
    int cur = 0;
    if (hipGetDevice(&cur) == hipSuccess && hipSetDevice(kv.first.first) == hipSuccess) {
      // The buffer's own stream may no longer exist: wait for the whole
      // device, then free on the null stream and wait for that.
      (void)hipDeviceSynchronize();
      (void)hipFreeAsync(kv.second.buf, nullptr);
      (void)hipDeviceSynchronize();
      (void)hipSetDevice(cur);
    }
  }
  g_scratch.clear();
}

}  // extern "C"
