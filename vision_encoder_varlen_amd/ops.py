"""PyTorch-facing wrappers over the C ABI of libvit.so.

Argument marshalling only: every step runs in the library's HIP kernels.
PyTorch provides device memory and the current stream.  Errors from the
library raise ``VitError`` (a ``ValueError``) carrying its message.
"""
from __future__ import annotations

import math
from typing import Optional, Tuple

import torch

from . import _lib

_DTYPES = {torch.float32: _lib.VIT_F32, torch.bfloat16: _lib.VIT_BF16}


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _need_cuda(name: str, t: torch.Tensor, dtype=None, token_strided: bool = False) -> None:
    """CUDA tensor of ``dtype``; contiguous, or (``token_strided``) a ``[T, H, D]``
    view whose heads are contiguous within a token (any token stride)."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if token_strided and t.dim() == 3:
        _, H, D = t.shape
        if t.stride(2) != 1 or t.stride(1) != D:
            raise ValueError(f"{name}: the heads of a token must be contiguous ([T, H, D] view)")
    elif not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def _strides(*ts: torch.Tensor):
    """ctypes int64 array of the tensors' token strides, or None when all are dense."""
    import ctypes
    vals = [t.stride(0) if t.shape[0] > 1 else t.shape[1] * t.shape[2] for t in ts]
    if all(v == t.shape[1] * t.shape[2] for v, t in zip(vals, ts)):
        return None
    return (ctypes.c_int64 * len(vals))(*vals)


def _strides_qk(q, k):
    """Token strides of (q, k) for the pre-pass; q may be None (k only)."""
    return _strides(k, k) if q is None else _strides(q, k)


def dtype_code(dtype: torch.dtype) -> int:
    if dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {dtype}; expected float32 or bfloat16")
    return _DTYPES[dtype]


def _prepass_checks(q, k, pos, q_weight, k_weight) -> None:
    if q is not None:
        _need_cuda("q", q, token_strided=True)
    _need_cuda("k", k, None if q is None else q.dtype, token_strided=True)
    if k.dim() != 3 or (q is not None and k.shape != q.shape):
        raise ValueError("q and k must both be [T, H, D]")
    T, H, D = k.shape
    if pos is not None:
        _need_cuda("pos", pos, torch.int32)
        if pos.shape != (T, 2):
            raise ValueError("pos must be int32 [T, 2]")
    for name, w in (("q_weight", q_weight), ("k_weight", k_weight)):
        if w is not None:
            _need_cuda(name, w, torch.float32)
            if w.shape != (D,):
                raise ValueError(f"{name} must be float32 [D]")


_ROPE_MODES = {"neox": _lib.VIT_ROPE_NEOX, "complex": _lib.VIT_ROPE_COMPLEX}


def _rope_mode(mode: str) -> int:
    if mode not in _ROPE_MODES:
        raise ValueError(f"unknown rope mode {mode!r}; expected 'neox' or 'complex'")
    return _ROPE_MODES[mode]


def qk_norm_rope_(q: torch.Tensor, k: torch.Tensor, pos: Optional[torch.Tensor] = None,
                  theta: float = 10000.0, q_weight: Optional[torch.Tensor] = None,
                  k_weight: Optional[torch.Tensor] = None, eps: float = 1e-6,
                  rope_mode: str = "neox") -> None:
    """In-place Q/K RMSNorm (when weights are given) then 2D rotary (when ``pos`` is given).

    ``rope_mode``: ``"neox"`` pairs ``(m, m + D/2)``; ``"complex"`` pairs ``(2j, 2j + 1)``.
    ``q`` may be None (k only; q's half then runs inside ``varlen_attn_planned_qnorm_rope``)."""
    _prepass_checks(q, k, pos, q_weight, k_weight)
    T, H, D = k.shape
    _lib.check(_lib.load().vit_qk_norm_rope_ex(
        _ptr(q), k.data_ptr(), T, H, D, dtype_code(k.dtype), _ptr(pos), float(theta),
        _ptr(q_weight), _ptr(k_weight), float(eps), _rope_mode(rope_mode), _strides_qk(q, k),
        _stream(k)))


def qk_norm_rope_worklist_(q: torch.Tensor, k: torch.Tensor, pos: Optional[torch.Tensor],
                           theta: float, q_weight: Optional[torch.Tensor],
                           k_weight: Optional[torch.Tensor], eps: float, plan: "Plan",
                           cu_seqlens: torch.Tensor, rope_mode: str = "neox") -> "Plan":
    """``qk_norm_rope_`` and ``rebuild_worklist(plan, cu_seqlens)`` in one launch."""
    _prepass_checks(q, k, pos, q_weight, k_weight)
    _need_cuda("cu_seqlens", cu_seqlens, torch.int32)
    if cu_seqlens.numel() - 1 != plan.num_seqs:
        raise ValueError("cu_seqlens does not match the plan")
    T, H, D = k.shape
    _lib.check(_lib.load().vit_qk_norm_rope_worklist(
        _ptr(q), k.data_ptr(), T, H, D, dtype_code(k.dtype), _ptr(pos), float(theta),
        _ptr(q_weight), _ptr(k_weight), float(eps), _rope_mode(rope_mode), _strides_qk(q, k),
        cu_seqlens.data_ptr(), plan.num_seqs,
        plan.max_seqlen, plan.block_m, plan.items.data_ptr(), plan.cap, plan.meta.data_ptr(),
        _stream(k)))
    return plan


def qk_norm_rope_into(q_src: Optional[torch.Tensor], k_src: torch.Tensor,
                      q: Optional[torch.Tensor], k: torch.Tensor, pos: Optional[torch.Tensor],
                      theta: float = 10000.0, q_weight: Optional[torch.Tensor] = None,
                      k_weight: Optional[torch.Tensor] = None, eps: float = 1e-6,
                      rope_mode: str = "neox", plan: Optional["Plan"] = None,
                      cu_seqlens: Optional[torch.Tensor] = None) -> None:
    """Q/K RMSNorm then 2D rotary from ``q_src`` / ``k_src`` (left unchanged)
    into ``q`` / ``k``; with ``plan`` and ``cu_seqlens`` the plan's work-list
    is rebuilt in the same launch.  An output is either its own source (in
    place) or shares no memory with the sources."""
    _prepass_checks(q, k, pos, q_weight, k_weight)
    if (q_src is None) != (q is None):
        raise ValueError("q_src and q must both be given or both be None")
    if q_src is not None:
        _need_cuda("q_src", q_src, q.dtype, token_strided=True)
        if q_src.shape != q.shape:
            raise ValueError("q_src must have the shape of q")
    _need_cuda("k_src", k_src, k.dtype, token_strided=True)
    if k_src.shape != k.shape:
        raise ValueError("k_src must have the shape of k")
    if (plan is None) != (cu_seqlens is None):
        raise ValueError("give plan and cu_seqlens together")
    if plan is not None:
        _need_cuda("cu_seqlens", cu_seqlens, torch.int32)
        if cu_seqlens.numel() - 1 != plan.num_seqs:
            raise ValueError("cu_seqlens does not match the plan")
    T, H, D = k.shape
    lst = (None, 0, 0, 0, None, 0, None) if plan is None else (
        cu_seqlens.data_ptr(), plan.num_seqs, plan.max_seqlen, plan.block_m, plan.items.data_ptr(),
        plan.cap, plan.meta.data_ptr())
    _lib.check(_lib.load().vit_qk_norm_rope_into(
        _ptr(q_src), k_src.data_ptr(), _strides_qk(q_src, k_src), _ptr(q), k.data_ptr(), T, H, D,
        dtype_code(k.dtype), _ptr(pos), float(theta), _ptr(q_weight), _ptr(k_weight), float(eps),
        _rope_mode(rope_mode), _strides_qk(q, k), *lst, _stream(k)))


def _attn_checks(q, k, v, cu_seqlens):
    _need_cuda("q", q, token_strided=True)
    for name, t in (("k", k), ("v", v)):
        _need_cuda(name, t, q.dtype, token_strided=True)
        if t.shape != q.shape:
            raise ValueError(f"{name} must have the shape of q")
    if q.dim() != 3:
        raise ValueError("q must be [T, H, D]")
    _need_cuda("cu_seqlens", cu_seqlens, torch.int32)
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens must be int32 [N+1]")


def varlen_attn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens: torch.Tensor,
                max_seqlen: int, scale: Optional[float] = None,
                out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                causal: bool = False) -> torch.Tensor:
    """Block-diagonal attention over packed ``[T, H, D]`` tensors (non-causal
    unless ``causal``: then query ``a`` of a segment sees keys ``0..a`` of it).

    ``scale`` defaults to ``head_dim ** -0.5``.  Dispatches on dtype: bf16 uses
    the MFMA kernel, fp32 the fp32 kernel.  ``lse`` (optional, fp32 ``[T, H]``)
    receives each row's log-sum-exp of scores.  Returns ``out``.
    """
    _attn_checks(q, k, v, cu_seqlens)
    T, H, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    else:
        _need_cuda("out", out, q.dtype, token_strided=True)
        if out.shape != q.shape:
            raise ValueError("out must have the shape of q")
    if lse is not None:
        _need_cuda("lse", lse, torch.float32)
        if lse.shape != (T, H):
            raise ValueError("lse must be float32 [T, H]")
    lib = _lib.load()
    strides = _strides(q, k, v, out)
    if lse is not None or strides is not None or causal:
        _lib.check(lib.vit_varlen_attn_ex(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), cu_seqlens.data_ptr(), cu_seqlens.numel() - 1,
            int(max_seqlen), H, D, float(scale), dtype_code(q.dtype), _flags(causal),
            out.data_ptr(), _ptr(lse), strides, _stream(q)))
        return out
    fn = lib.vit_varlen_attn if q.dtype == torch.bfloat16 else lib.vit_varlen_attn_f32
    dtype_code(q.dtype)
    _lib.check(fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), cu_seqlens.data_ptr(),
                  cu_seqlens.numel() - 1, int(max_seqlen), H, D, float(scale), out.data_ptr(),
                  _stream(q)))
    return out


def varlen_attn_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                        cu_seqlens: torch.Tensor, max_seqlen: int, out: torch.Tensor,
                        scale: Optional[float] = None, lse: Optional[torch.Tensor] = None,
                        causal: bool = False) -> torch.Tensor:
    """``varlen_attn`` through ``vit_varlen_attn_noalloc``: the work-list goes to
    the library's fixed device array, so nothing is allocated (``out`` must be
    given).  Calls that overlap in time on one GPU race on that array."""
    _attn_checks(q, k, v, cu_seqlens)
    T, H, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    _need_cuda("out", out, q.dtype, token_strided=True)
    if out.shape != q.shape:
        raise ValueError("out must have the shape of q")
    if lse is not None:
        _need_cuda("lse", lse, torch.float32)
        if lse.shape != (T, H):
            raise ValueError("lse must be float32 [T, H]")
    _lib.check(_lib.load().vit_varlen_attn_noalloc(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), cu_seqlens.data_ptr(), cu_seqlens.numel() - 1,
        int(max_seqlen), H, D, float(scale), dtype_code(q.dtype), _flags(causal), out.data_ptr(),
        _ptr(lse), _strides(q, k, v, out), _stream(q)))
    return out


def _flags(causal: bool) -> int:
    return _lib.VIT_ATTN_CAUSAL if causal else 0


def dense_batch_attn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, batch: int, seq_len: int,
                     scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                     lse: Optional[torch.Tensor] = None, causal: bool = False) -> torch.Tensor:
    """Attention over a uniform batch of ``batch`` segments of ``seq_len`` tokens
    (``cu_seqlens = None``), packed ``[batch * seq_len, H, D]``.  No work-list,
    no metadata, no allocation beyond ``out`` when it is not given."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need_cuda(name, t, q.dtype, token_strided=True)
        if t.dim() != 3 or t.shape != q.shape:
            raise ValueError(f"{name} must be [batch * seq_len, H, D] like q")
    T, H, D = q.shape
    if T != int(batch) * int(seq_len):
        raise ValueError(f"q has {T} tokens, expected batch * seq_len = {int(batch) * int(seq_len)}")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    else:
        _need_cuda("out", out, q.dtype, token_strided=True)
        if out.shape != q.shape:
            raise ValueError("out must have the shape of q")
    if lse is not None:
        _need_cuda("lse", lse, torch.float32)
        if lse.shape != (T, H):
            raise ValueError("lse must be float32 [T, H]")
    _lib.check(_lib.load().vit_dense_batch_attn(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), int(batch), int(seq_len), H, D, float(scale),
        dtype_code(q.dtype), _flags(causal), out.data_ptr(), _ptr(lse), _strides(q, k, v, out),
        _stream(q)))
    return out


def attn_block_m(num_heads: int, head_dim: int, dtype: torch.dtype) -> int:
    bm = _lib.load().vit_attn_block_m(num_heads, head_dim, dtype_code(dtype))
    if bm < 0:
        _lib.check(-bm)
    return bm


def worklist_capacity(num_seqs: int, max_seqlen: int, block_m: int) -> int:
    return int(_lib.load().vit_worklist_capacity(num_seqs, max_seqlen, block_m))


class Plan:
    """A device work-list for one ``cu_seqlens``, reusable across layers."""

    def __init__(self, items: torch.Tensor, meta: torch.Tensor, cap: int, block_m: int,
                 num_seqs: int, max_seqlen: int):
        self.items, self.meta, self.cap, self.block_m = items, meta, cap, block_m
        self.num_seqs, self.max_seqlen = num_seqs, max_seqlen


def varlen_worklist(cu_seqlens: torch.Tensor, max_seqlen: int, block_m: int,
                    cap: Optional[int] = None) -> Plan:
    """Build the longest-first (segment, q-tile) list on the device."""
    _need_cuda("cu_seqlens", cu_seqlens, torch.int32)
    n = cu_seqlens.numel() - 1
    need = worklist_capacity(n, int(max_seqlen), int(block_m))
    if need < 0:
        raise ValueError("bad work-list sizes")
    cap = need if cap is None else int(cap)
    # (segment, q-tile, first token, length) per item; torch's allocations are
    # 256-byte aligned, which the 16-byte item reads need.
    items = torch.empty((max(cap, 1), 4), dtype=torch.int32, device=cu_seqlens.device)
    meta = torch.empty(2, dtype=torch.int32, device=cu_seqlens.device)
    _lib.check(_lib.load().vit_varlen_worklist(
        cu_seqlens.data_ptr(), n, int(max_seqlen), int(block_m), items.data_ptr(), cap,
        meta.data_ptr(), _stream(cu_seqlens)))
    return Plan(items, meta, cap, int(block_m), n, int(max_seqlen))


def rebuild_worklist(plan: Plan, cu_seqlens: torch.Tensor) -> Plan:
    """Rebuild ``plan`` in place for new ``cu_seqlens`` with the same segment count
    and ``max_seqlen`` bound (no allocation)."""
    _need_cuda("cu_seqlens", cu_seqlens, torch.int32)
    if cu_seqlens.numel() - 1 != plan.num_seqs:
        raise ValueError("cu_seqlens has a different segment count than the plan")
    _lib.check(_lib.load().vit_varlen_worklist(
        cu_seqlens.data_ptr(), plan.num_seqs, plan.max_seqlen, plan.block_m, plan.items.data_ptr(),
        plan.cap, plan.meta.data_ptr(), _stream(cu_seqlens)))
    return plan


def _check_plan_span(plan: "Plan", k: torch.Tensor, v: torch.Tensor) -> None:
    """The bf16 kernel addresses one segment's k and v rows with 32-bit byte
    offsets, counted with the key padding of its last tile (64 rows): a segment
    whose span exceeds 2^30 bytes would be skipped without an error, so the
    plan's length bound must keep every listed segment inside it.  (The list
    holds no segment longer than ``plan.max_seqlen``.)  The bound is the one
    the C ABI applies to ``max_seqlen`` for both dtypes."""
    stride = max(int(k.stride(0)), int(v.stride(0)))
    if (int(plan.max_seqlen) + 64) * stride * 2 > (1 << 30):
        raise ValueError(f"plan.max_seqlen {plan.max_seqlen} with token stride {stride}: a segment's "
                         "k/v rows would exceed the kernel's 2^30-byte addressing span")


def varlen_attn_planned(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                        cu_seqlens: torch.Tensor, plan: Plan, scale: Optional[float] = None,
                        out: Optional[torch.Tensor] = None,
                        lse: Optional[torch.Tensor] = None, causal: bool = False) -> torch.Tensor:
    """Attention over a work-list from ``varlen_worklist`` (built with ``attn_block_m``)."""
    _attn_checks(q, k, v, cu_seqlens)
    T, H, D = q.shape
    if plan.block_m != attn_block_m(H, D, q.dtype):
        raise ValueError("plan was built with a different block_m than this kernel uses")
    _check_plan_span(plan, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    else:
        _need_cuda("out", out, q.dtype, token_strided=True)
        if out.shape != q.shape:
            raise ValueError("out must have the shape of q")
    if lse is not None:
        _need_cuda("lse", lse, torch.float32)
        if lse.shape != (T, H):
            raise ValueError("lse must be float32 [T, H]")
    _lib.check(_lib.load().vit_varlen_attn_planned(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), cu_seqlens.data_ptr(), plan.items.data_ptr(),
        plan.cap, plan.meta.data_ptr(), H, D, float(scale), dtype_code(q.dtype), _flags(causal),
        out.data_ptr(), _ptr(lse), _strides(q, k, v, out), _stream(q)))
    return out


def varlen_attn_planned_qnorm_rope(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                                   cu_seqlens: torch.Tensor, plan: Plan,
                                   pos: Optional[torch.Tensor], theta: float = 10000.0,
                                   q_weight: Optional[torch.Tensor] = None, eps: float = 1e-6,
                                   rope_mode: str = "neox", scale: Optional[float] = None,
                                   out: Optional[torch.Tensor] = None,
                                   lse: Optional[torch.Tensor] = None,
                                   causal: bool = False) -> torch.Tensor:
    """``varlen_attn_planned`` with q's RMSNorm + rotary applied inside the kernel
    (``q`` itself is left unchanged); prepare ``k`` with ``qk_norm_rope_(None, k, ...)``."""
    _attn_checks(q, k, v, cu_seqlens)
    T, H, D = q.shape
    if plan.block_m != attn_block_m(H, D, q.dtype):
        raise ValueError("plan was built with a different block_m than this kernel uses")
    _check_plan_span(plan, k, v)
    if pos is not None:
        _need_cuda("pos", pos, torch.int32)
        if pos.shape != (T, 2):
            raise ValueError("pos must be int32 [T, 2]")
    if q_weight is not None:
        _need_cuda("q_weight", q_weight, torch.float32)
        if q_weight.shape != (D,):
            raise ValueError("q_weight must be float32 [D]")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    else:
        _need_cuda("out", out, q.dtype, token_strided=True)
        if out.shape != q.shape:
            raise ValueError("out must have the shape of q")
    if lse is not None:
        _need_cuda("lse", lse, torch.float32)
        if lse.shape != (T, H):
            raise ValueError("lse must be float32 [T, H]")
    _lib.check(_lib.load().vit_varlen_attn_planned_qnorm_rope(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), cu_seqlens.data_ptr(), plan.items.data_ptr(),
        plan.cap, plan.meta.data_ptr(), H, D, float(scale), dtype_code(q.dtype), _flags(causal),
        _ptr(pos), float(theta), _ptr(q_weight), float(eps), _rope_mode(rope_mode),
        out.data_ptr(), _ptr(lse), _strides(q, k, v, out), _stream(q)))
    return out


def varlen_attn_planned_qk_norm_rope(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                                     cu_seqlens: torch.Tensor, plan: Plan,
                                     pos: Optional[torch.Tensor], theta: float = 10000.0,
                                     q_weight: Optional[torch.Tensor] = None,
                                     k_weight: Optional[torch.Tensor] = None, eps: float = 1e-6,
                                     rope_mode: str = "neox", scale: Optional[float] = None,
                                     out: Optional[torch.Tensor] = None,
                                     lse: Optional[torch.Tensor] = None,
                                     causal: bool = False) -> torch.Tensor:
    """``varlen_attn_planned`` with the RMSNorm + rotary of both q and k applied
    inside the kernel (q and k themselves are left unchanged): no separate
    pre-pass.  ``q_weight`` and ``k_weight`` are both given or both None."""
    _attn_checks(q, k, v, cu_seqlens)
    T, H, D = q.shape
    if plan.block_m != attn_block_m(H, D, q.dtype):
        raise ValueError("plan was built with a different block_m than this kernel uses")
    _check_plan_span(plan, k, v)
    if pos is not None:
        _need_cuda("pos", pos, torch.int32)
        if pos.shape != (T, 2):
            raise ValueError("pos must be int32 [T, 2]")
    if (q_weight is None) != (k_weight is None):
        raise ValueError("q_weight and k_weight must both be given or both be None")
    for name, w in (("q_weight", q_weight), ("k_weight", k_weight)):
        if w is not None:
            _need_cuda(name, w, torch.float32)
            if w.shape != (D,):
                raise ValueError(f"{name} must be float32 [D]")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    else:
        _need_cuda("out", out, q.dtype, token_strided=True)
        if out.shape != q.shape:
            raise ValueError("out must have the shape of q")
    if lse is not None:
        _need_cuda("lse", lse, torch.float32)
        if lse.shape != (T, H):
            raise ValueError("lse must be float32 [T, H]")
    _lib.check(_lib.load().vit_varlen_attn_planned_qk_norm_rope(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), cu_seqlens.data_ptr(), plan.items.data_ptr(),
        plan.cap, plan.meta.data_ptr(), H, D, float(scale), dtype_code(q.dtype), _flags(causal),
        _ptr(pos), float(theta), _ptr(q_weight), _ptr(k_weight), float(eps),
        _rope_mode(rope_mode), out.data_ptr(), _ptr(lse), _strides(q, k, v, out), _stream(q)))
    return out


def device_error(reset: bool = False, device: Optional[torch.device] = None) -> int:
    """Work-list error bits of the last ``varlen_attn`` on the current stream (syncs it)."""
    import ctypes
    stream = torch.cuda.current_stream(device).cuda_stream
    err = ctypes.c_int32(0)
    _lib.check(_lib.load().vit_device_error(stream, ctypes.byref(err), int(bool(reset))))
    return int(err.value)


def release() -> None:
    _lib.load().vit_release()


def time_next_kernel(start: Optional["torch.cuda.Event"], stop: Optional["torch.cuda.Event"]) -> None:
    """Have the next kernel-launching call of this module on this thread record
    ``start``/``stop`` at its kernel's dispatch start and end (for the attention
    calls: the attention kernel).  Events need ``enable_timing=True``;
    ``None, None`` clears the hook."""
    if start is None and stop is None:
        _lib.check(_lib.load().vit_time_next_kernel(None, None))
        return
    for ev in (start, stop):
        if ev.cuda_event == 0:     # torch creates the HIP event on first record
            ev.record()
    _lib.check(_lib.load().vit_time_next_kernel(start.cuda_event, stop.cuda_event))
