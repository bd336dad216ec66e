"""Fused RMSNorm + 2D RoPE kernel vs the fp64 oracle."""
import numpy as np
import pytest

import oracle
from vision_encoder_varlen_amd import workloads as W
from gpu_util import assert_prepass_close, to_dev, to_host

pytestmark = pytest.mark.gpu


def _run(wl, rope=True, norm=None, theta=10000.0, rope_mode="neox"):
    import torch
    from vision_encoder_varlen_amd import ops
    x = W.generate(wl)
    norm = wl.use_norm if norm is None else norm
    q, k = to_dev(x.q, wl.dtype), to_dev(x.k, wl.dtype)
    pos = torch.from_numpy(x.pos).cuda() if rope else None
    wq = torch.from_numpy(x.wq).cuda() if norm else None
    wk = torch.from_numpy(x.wk).cuda() if norm else None
    ops.qk_norm_rope_(q, k, pos, theta, wq, wk, wl.eps, rope_mode=rope_mode)
    torch.cuda.synchronize()
    eq, ek = oracle.qk_norm_rope(x.q, x.k, x.pos if rope else None, theta,
                                 x.wq if norm else None, x.wk if norm else None, wl.eps,
                                 rope_mode=rope_mode)
    return to_host(q), to_host(k), eq, ek, x


@pytest.mark.parametrize("D", [32, 64, 80, 96, 128])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("norm", [False, True])
def test_prepass_matches_oracle(D, dtype, norm):
    wl = W.custom([(4, 4), (6, 8), (1, 1), (13, 7), (64, 2)], H=3, D=D, dtype=dtype, seed=D + norm)
    gq, gk, eq, ek, _ = _run(wl, rope=True, norm=norm)
    assert_prepass_close(gq, eq, dtype, f"q D={D}")
    assert_prepass_close(gk, ek, dtype, f"k D={D}")


@pytest.mark.parametrize("D", [64, 128])
def test_norm_only(D):
    wl = W.custom([(5, 9), (3, 3)], H=4, D=D, dtype="bf16", seed=3, use_norm=True)
    gq, gk, eq, ek, _ = _run(wl, rope=False, norm=True)
    assert_prepass_close(gq, eq, "bf16", "q norm only")
    assert_prepass_close(gk, ek, "bf16", "k norm only")


def test_origin_is_bit_exact_identity_without_norm():
    wl = W.custom([(1, 1)] * 37, H=5, D=128, dtype="bf16", seed=4)  # every token at (0, 0)
    gq, gk, _, _, x = _run(wl, rope=True, norm=False)
    assert np.array_equal(gq, x.q.astype(np.float64))
    assert np.array_equal(gk, x.k.astype(np.float64))


def test_other_theta_and_large_positions():
    wl = W.custom([(128, 128)], H=2, D=64, dtype="f32", seed=9)
    gq, gk, eq, ek, _ = _run(wl, rope=True, norm=False, theta=500.0)
    assert_prepass_close(gq, eq, "f32", "q theta=500")
    assert_prepass_close(gk, ek, "f32", "k theta=500")


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
def test_workload_prepass_sampled_tokens(n):
    """Full-size workloads, in the launch configuration the benchmark uses; the
    pre-pass is per token, so the oracle checks a random sample of tokens."""
    import torch
    from vision_encoder_varlen_amd import ops
    wl = W.config(n)
    x = W.generate(wl)
    q, k = to_dev(x.q, wl.dtype), to_dev(x.k, wl.dtype)
    pos = torch.from_numpy(x.pos).cuda()
    wq = torch.from_numpy(x.wq).cuda() if wl.use_norm else None
    wk = torch.from_numpy(x.wk).cuda() if wl.use_norm else None
    ops.qk_norm_rope_(q, k, pos, wl.theta, wq, wk, wl.eps)
    torch.cuda.synchronize()
    rng = np.random.default_rng(77 + n)
    idx = np.unique(np.concatenate([rng.integers(0, wl.total_tokens, size=2048),
                                    [0, wl.total_tokens - 1]]))
    eq, ek = oracle.qk_norm_rope(x.q[idx], x.k[idx], x.pos[idx], wl.theta,
                                 x.wq if wl.use_norm else None, x.wk if wl.use_norm else None, wl.eps)
    it = torch.from_numpy(idx).cuda()
    assert_prepass_close(to_host(q[it]), eq, wl.dtype, f"config {n} q")
    assert_prepass_close(to_host(k[it]), ek, wl.dtype, f"config {n} k")


@pytest.mark.parametrize("D", [8, 32, 64, 80, 96, 128, 256])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("norm", [False, True])
def test_complex_rope_matches_oracle(D, dtype, norm):
    """Complex-form rotary (pairs (2j, 2j+1)), with and without the norm."""
    wl = W.custom([(4, 4), (6, 8), (1, 1), (13, 7), (64, 2)], H=3, D=D, dtype=dtype, seed=D + 7)
    gq, gk, eq, ek, _ = _run(wl, rope=True, norm=norm, rope_mode="complex")
    assert_prepass_close(gq, eq, dtype, f"complex q D={D}")
    assert_prepass_close(gk, ek, dtype, f"complex k D={D}")


def test_complex_rope_fused_with_worklist_and_strided():
    """The complex mode through the fused pre-pass + work-list launch on packed
    [T, 3, H, D] views equals the plain call on contiguous tensors, bit for bit."""
    import torch
    from vision_encoder_varlen_amd import ops
    wl = W.custom([(6, 8), (17, 5), (32, 32)], H=2, D=64, dtype="bf16", seed=12, use_norm=True)
    x = W.generate(wl)
    qkv = torch.stack([to_dev(a, "bf16") for a in (x.q, x.k, x.v)], dim=1)
    q, k = qkv[:, 0], qkv[:, 1]
    qd, kd = q.contiguous(), k.contiguous()
    pos = torch.from_numpy(x.pos).cuda()
    wq, wk = torch.from_numpy(x.wq).cuda(), torch.from_numpy(x.wk).cuda()
    cu = torch.from_numpy(x.cu_seqlens).cuda()
    plan = ops.varlen_worklist(cu, wl.max_seqlen, ops.attn_block_m(wl.H, wl.D, q.dtype))
    ops.qk_norm_rope_(qd, kd, pos, wl.theta, wq, wk, wl.eps, rope_mode="complex")
    ops.qk_norm_rope_worklist_(q, k, pos, wl.theta, wq, wk, wl.eps, plan, cu, rope_mode="complex")
    torch.cuda.synchronize()
    assert torch.equal(q, qd) and torch.equal(k, kd)
    eq, ek = oracle.qk_norm_rope(x.q, x.k, x.pos, wl.theta, x.wq, x.wk, wl.eps, rope_mode="complex")
    assert_prepass_close(to_host(q), eq, "bf16", "complex fused q")
    assert_prepass_close(to_host(k), ek, "bf16", "complex fused k")
    with pytest.raises(ValueError):
        ops.qk_norm_rope_(qd, kd, pos, rope_mode="gptj")
