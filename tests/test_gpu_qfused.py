"""The Q half of the pre-pass inside the attention kernel
(vit_varlen_attn_planned_qnorm_rope) with a k-only pre-pass, through the C ABI.

* the k-only pre-pass writes exactly what the full pre-pass writes to k, and
  leaves q alone;
* the fused attention leaves q unchanged in memory;
* its output matches the oracle's end-to-end result (fp64 pre-pass rounded
  once to the storage dtype, then attention) within the attention tolerance,
  for every head dim, both dtypes, both rotary pairings, with and without the
  norm, and the causal flag;
* full-size workloads, every element, in the launch configuration the
  benchmark's fused step uses.
"""
import numpy as np
import pytest

import oracle
from vision_encoder_varlen_amd import workloads as W
from gpu_util import assert_attn_close, to_dev, to_host, workload_oracle

pytestmark = pytest.mark.gpu

GRIDS = [(4, 4), (6, 8), (1, 1), (13, 7), (64, 2), (20, 15)]


def _fused(wl, x, rope_mode="neox", causal=False):
    import torch
    from vision_encoder_varlen_amd import ops
    q, k, v = (to_dev(a, wl.dtype) for a in (x.q, x.k, x.v))
    q0 = q.clone()
    pos = torch.from_numpy(x.pos).cuda()
    cu = torch.from_numpy(x.cu_seqlens).cuda()
    wq = torch.from_numpy(x.wq).cuda() if wl.use_norm else None
    wk = torch.from_numpy(x.wk).cuda() if wl.use_norm else None
    # reference k: the full pre-pass on a copy
    qr, kr = q.clone(), k.clone()
    ops.qk_norm_rope_(qr, kr, pos, wl.theta, wq, wk, wl.eps, rope_mode=rope_mode)
    ops.qk_norm_rope_(None, k, pos, wl.theta, None, wk, wl.eps, rope_mode=rope_mode)
    plan = ops.varlen_worklist(cu, wl.max_seqlen, ops.attn_block_m(wl.H, wl.D, q.dtype))
    out = ops.varlen_attn_planned_qnorm_rope(q, k, v, cu, plan, pos, wl.theta, wq, wl.eps,
                                             rope_mode, causal=causal)
    ref = ops.varlen_attn_planned(qr, kr, v, cu, plan, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(k, kr), "the k-only pre-pass differs from the k half of the full one"
    assert torch.equal(q, q0), "the fused attention modified q"
    return to_host(out), to_host(ref)


def _want(wl, x, rope_mode="neox", causal=False):
    norm_w = (x.wq, x.wk) if wl.use_norm else (None, None)
    eq, ek = oracle.qk_norm_rope(x.q, x.k, x.pos, wl.theta, *norm_w, wl.eps, rope_mode=rope_mode)
    eq, ek = oracle.round_to_dtype(eq, wl.dtype), oracle.round_to_dtype(ek, wl.dtype)
    return oracle.varlen_attention(eq, ek, x.v, x.cu_seqlens, wl.softmax_scale, causal=causal)


@pytest.mark.parametrize("D", [32, 64, 80, 96, 128])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("norm", [False, True])
@pytest.mark.parametrize("rope_mode", ["neox", "complex"])
def test_fused_q_matches_oracle(D, dtype, norm, rope_mode):
    wl = W.custom(GRIDS, H=3, D=D, dtype=dtype, seed=90 + D, use_norm=norm)
    x = W.generate(wl)
    got, ref = _fused(wl, x, rope_mode)
    want = _want(wl, x, rope_mode)
    assert_attn_close(got, want, dtype, f"fused q D={D} {dtype} norm={norm} {rope_mode}")
    assert_attn_close(ref, want, dtype, "separate pre-pass")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_fused_q_causal(dtype):
    wl = W.custom(GRIDS, H=2, D=64, dtype=dtype, seed=95, use_norm=True)
    x = W.generate(wl)
    got, _ = _fused(wl, x, causal=True)
    assert_attn_close(got, _want(wl, x, causal=True), dtype, "fused q causal", peaked=True)


def test_fused_q_large_positions_and_theta():
    """A 96 x 96 grid (coordinates up to 95): the angle is reduced exactly
    before the hardware sine and cosine."""
    wl = W.custom([(96, 96)], H=2, D=128, dtype="bf16", seed=96, use_norm=True)
    x = W.generate(wl)
    got, _ = _fused(wl, x)
    assert_attn_close(got, _want(wl, x), "bf16", "fused q 96x96")


@pytest.mark.parametrize("D", [64, 80, 128])
@pytest.mark.parametrize("rope_mode", ["neox", "complex"])
def test_fused_q_positions_outside_the_table(D, rope_mode):
    """Negative coordinates and coordinates of 64 and more next to small
    ones: waves with any of them evaluate the angles directly, the others read
    the workgroup's table."""
    wl = W.custom([(10, 13), (7, 9), (3, 40)], H=2, D=D, dtype="bf16", seed=97, use_norm=True)
    x = W.generate(wl)
    rng = np.random.default_rng(97)
    pos = x.pos.astype(np.int64)
    pos[:130] += rng.integers(-200, 200, size=(130, 2))
    pos[193:] = rng.integers(60, 70, size=(wl.total_tokens - 193, 2))
    x.pos = pos.astype(np.int32)
    got, _ = _fused(wl, x, rope_mode)
    assert_attn_close(got, _want(wl, x, rope_mode), "bf16", f"fused q positions D={D}")


@pytest.mark.parametrize("n", [2, 3])
def test_fused_q_workload(n):
    """4 x (32 x 32) at D = 80, and the 24-image ragged batch at D = 128 with
    the norm: every element against the oracle's end-to-end result."""
    wl = W.config(n)
    x = W.generate(wl)
    got, _ = _fused(wl, x)
    assert_attn_close(got, workload_oracle(n, "e2e"), wl.dtype, f"config {n} fused q")
