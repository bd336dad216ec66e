// Varlen (block-diagonal) attention, bf16 in/out, for gfx950: launches of the
// plain kernels (no pre-pass inside; see attn_bf16_kernel.h for the design).
// Calls asking for part of the pre-pass go to attn_bf16_fused.hip.
#include "attn_bf16_kernel.h"

namespace vit {
namespace {

template <int D>
hipError_t launch_d(const void* q, const void* k, const void* v, const Schedule& sch, int H,
                    float scale, bool causal, const QPrepass* qp, void* out, float* lse,
                    TokenStrides ts, hipStream_t stream, hipEvent_t e0, hipEvent_t e1) {
  using C = typename Choice<D>::C;
  static_assert(C::BM == bf16_block_m_const(D), "work-list block size mismatch");
  return launch_cfg<C>(q, k, v, sch, H, scale, causal, qp, out, lse, ts, stream, e0, e1);
}

}  // namespace

hipError_t launch_attn_bf16(const void* q, const void* k, const void* v, const Schedule& sch,
                            int H, int D, float scale, bool causal, const QPrepass* qp, void* out,
                            float* lse, TokenStrides ts, hipStream_t stream, hipEvent_t e0,
                            hipEvent_t e1) {
  if (qp != nullptr && (qp->fuse_k || qp->pos != nullptr || qp->weight != nullptr))
    return launch_attn_bf16_fused(q, k, v, sch, H, D, scale, causal, qp, out, lse, ts, stream, e0,
                                  e1);
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
