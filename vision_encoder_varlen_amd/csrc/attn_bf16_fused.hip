// Varlen (block-diagonal) attention, bf16 in/out, for gfx950: launches of the
// kernels that do part of the pre-pass themselves (attn_bf16_kernel.h, PRE
// 1 and 2).  The RMSNorm and 2D rotary of _qkv_with_rope (vLLM page) are
// applied to q's rows as they are loaded (PRE 1, q only) and, with fuse_k,
// to every K tile in LDS as well (PRE 2), as the FA4 route on the tokenspeed
// page (MultimodalEncoderAttention.forward) fuses the rotary into the QKV
// split.  Every call that asks for any part of the pre-pass is launched
// from here; the plain kernels (PRE 0) still hold a direct query transform
// behind a runtime test, which these calls never reach.
#include "attn_bf16_kernel.h"

namespace vit {
namespace {

template <int D, int PRE>
hipError_t launch_pre(const void* q, const void* k, const void* v, const Schedule& sch, int H,
                      float scale, bool causal, const QPrepass* qp, void* out, float* lse,
                      TokenStrides ts, hipStream_t stream, hipEvent_t e0, hipEvent_t e1) {
  using C = typename Choice<D>::C::template WithPre<PRE>;
  static_assert(C::BM == bf16_block_m_const(D), "work-list block size mismatch");
  return launch_cfg<C>(q, k, v, sch, H, scale, causal, qp, out, lse, ts, stream, e0, e1);
}

template <int D>
hipError_t launch_d(const void* q, const void* k, const void* v, const Schedule& sch, int H,
                    float scale, bool causal, const QPrepass* qp, void* out, float* lse,
                    TokenStrides ts, hipStream_t stream, hipEvent_t e0, hipEvent_t e1) {
  return qp->fuse_k
             ? launch_pre<D, 2>(q, k, v, sch, H, scale, causal, qp, out, lse, ts, stream, e0, e1)
             : launch_pre<D, 1>(q, k, v, sch, H, scale, causal, qp, out, lse, ts, stream, e0, e1);
}

}  // namespace

hipError_t launch_attn_bf16_fused(const void* q, const void* k, const void* v, const Schedule& sch,
                                  int H, int D, float scale, bool causal, const QPrepass* qp,
                                  void* out, float* lse, TokenStrides ts, hipStream_t stream,
                                  hipEvent_t e0, hipEvent_t e1) {
  if (qp == nullptr) return hipErrorInvalidValue;
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
