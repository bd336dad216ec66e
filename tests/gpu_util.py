"""Helpers shared by the GPU parity tests (no test functions here)."""
from __future__ import annotations

import numpy as np

# Tolerances for attention outputs.  fp32: max-abs 1e-5.  bf16 (fp32
# accumulation): max-abs 1.5e-2 and relative L2 5e-3.
F32_MAX_ABS = 1e-5
BF16_MAX_ABS = 1.5e-2
BF16_REL_L2 = 5e-3


def torch_dtype(dtype: str):
    import torch
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def to_dev(x: np.ndarray, dtype: str):
    """float32 array holding exactly representable values -> device tensor of `dtype`."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch_dtype(dtype)).cuda()


def to_host(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def attn_errors(got: np.ndarray, want: np.ndarray):
    diff = got - want
    max_abs = float(np.max(np.abs(diff))) if diff.size else 0.0
    denom = float(np.linalg.norm(want))
    rel_l2 = float(np.linalg.norm(diff) / denom) if denom > 0 else float(np.linalg.norm(diff))
    return max_abs, rel_l2


def assert_attn_close(got: np.ndarray, want: np.ndarray, dtype: str, what: str = "",
                      peaked: bool = False):
    """peaked: rows that may return nearly single V rows (causal rows near a
    segment's start see only a few keys), whose magnitude can pass 4; there
    the bf16 weights P and the bf16 store each move an output by up to 2^-9
    of its size, so a bf16 element may differ by 1.5e-2 + 2^-8 |exact|."""
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    max_abs, rel_l2 = attn_errors(got, want)
    if dtype == "f32":
        assert max_abs <= F32_MAX_ABS, f"{what}: fp32 max-abs {max_abs:.3e} > {F32_MAX_ABS}"
    else:
        if peaked:
            err = np.abs(got - want)
            tol = BF16_MAX_ABS + 2.0 ** -8 * np.abs(want)
            worst = float((err / tol).max()) if err.size else 0.0
            assert worst <= 1.0, f"{what}: bf16 error {worst:.3f} of the magnitude-scaled bound"
        else:
            assert max_abs <= BF16_MAX_ABS, f"{what}: bf16 max-abs {max_abs:.3e} > {BF16_MAX_ABS}"
        assert rel_l2 <= BF16_REL_L2, f"{what}: bf16 rel-L2 {rel_l2:.3e} > {BF16_REL_L2}"
    return max_abs, rel_l2


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values at |x| (8 significant bits)."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(ax, np.finfo(np.float64).tiny)))
    return np.ldexp(1.0, (e - 7).astype(np.int64))


def assert_prepass_close(got: np.ndarray, exact: np.ndarray, dtype: str, what: str = ""):
    """fp32: max-abs 1e-5.

    bf16: |got - exact| <= ulp_bf16(|exact|) + 2^-20 * r, with r the length of the
    rotary pair (m, m + D/2) the element belongs to.  A correctly rounded result
    is within half an ulp; the kernel works in fp32, whose few roundings (norm
    factor, weight, cos/sin, the two products of the rotation) stay below
    16 * 2^-24 * r.  The second term only matters for results that cancel to
    nearly zero, where one bf16 ulp is smaller than fp32 noise on O(1) operands.
    """
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - exact)
    if dtype == "f32":
        assert float(err.max()) <= 1e-5, f"{what}: fp32 pre-pass max-abs {float(err.max()):.3e}"
    else:
        h = exact.shape[-1] // 2
        r = np.hypot(exact[..., :h], exact[..., h:])
        r = np.concatenate([r, r], axis=-1)
        tol = bf16_ulp(exact) + 2.0 ** -20 * r
        bad = err > tol
        assert not bad.any(), (f"{what}: {int(bad.sum())} bf16 elements beyond 1 ulp; "
                               f"worst {float((err / tol).max()):.2f} ulp")


# Oracle results for the seeded workloads, computed once per test process:
# several test modules compare against the same full-size results, and the
# largest (16384 tokens, 12 heads) costs the oracle tens of seconds.
_ORACLE_CACHE = {}


def workload_oracle(n: int, kind: str, causal: bool = False) -> np.ndarray:
    """Oracle output of seeded workload ``n`` (fp64 ``[T, H, D]``).

    kind "attn": attention alone on the seeded q, k, v.
    kind "e2e":  the oracle's fp64 pre-pass (norm when the workload has one,
                 then rotary), rounded once to the storage dtype, then attention.
    """
    import oracle
    from vision_encoder_varlen_amd import workloads as W
    key = (n, kind, causal)
    if key not in _ORACLE_CACHE:
        wl = W.config(n)
        x = W.generate(wl)
        if kind == "attn":
            q, k = x.q, x.k
        elif kind == "e2e":
            norm_w = (x.wq, x.wk) if wl.use_norm else (None, None)
            q, k = oracle.qk_norm_rope(x.q, x.k, x.pos, wl.theta, *norm_w, wl.eps)
            q, k = oracle.round_to_dtype(q, wl.dtype), oracle.round_to_dtype(k, wl.dtype)
        else:
            raise ValueError(kind)
        _ORACLE_CACHE[key] = oracle.varlen_attention(q, k, x.v, x.cu_seqlens, wl.softmax_scale,
                                                     causal=causal)
    return _ORACLE_CACHE[key]
