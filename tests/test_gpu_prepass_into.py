"""The out-of-place pre-pass (vit_qk_norm_rope_into) against the fp64 oracle.

The sources are read, never written: the outputs match the oracle, the
sources keep every bit, and the outputs equal the in-place call's bit for bit
(the same kernel reads the same rows).  Sources are views of a packed
[T, 3, H, D] buffer, as the QKV projection leaves them.
"""
import numpy as np
import pytest

import oracle
from vision_encoder_varlen_amd import workloads as W
from gpu_util import assert_prepass_close, to_dev, to_host

pytestmark = pytest.mark.gpu


def _inputs(wl):
    import torch
    x = W.generate(wl)
    qkv = torch.stack([to_dev(a, wl.dtype) for a in (x.q, x.k, x.v)], dim=1)
    pos = torch.from_numpy(x.pos).cuda()
    wq = torch.from_numpy(x.wq).cuda() if wl.use_norm else None
    wk = torch.from_numpy(x.wk).cuda() if wl.use_norm else None
    return x, qkv, pos, wq, wk


@pytest.mark.parametrize("D", [64, 80, 128])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("rope_mode", ["neox", "complex"])
def test_into_matches_oracle_and_keeps_sources(D, dtype, rope_mode):
    import torch
    from vision_encoder_varlen_amd import ops
    wl = W.custom([(4, 4), (6, 8), (1, 1), (13, 7), (64, 2)], H=3, D=D, dtype=dtype, seed=40 + D,
                  use_norm=True)
    x, qkv, pos, wq, wk = _inputs(wl)
    before = qkv.clone()
    q_src, k_src = qkv[:, 0], qkv[:, 1]
    q, k = torch.full_like(q_src.contiguous(), float("nan")), torch.full_like(k_src.contiguous(), float("nan"))
    ops.qk_norm_rope_into(q_src, k_src, q, k, pos, wl.theta, wq, wk, wl.eps, rope_mode=rope_mode)
    qi, ki = q_src.contiguous(), k_src.contiguous()
    ops.qk_norm_rope_(qi, ki, pos, wl.theta, wq, wk, wl.eps, rope_mode=rope_mode)
    torch.cuda.synchronize()
    assert torch.equal(qkv, before), "the sources changed"
    assert torch.equal(q, qi) and torch.equal(k, ki), "out of place differs from in place"
    eq, ek = oracle.qk_norm_rope(x.q, x.k, x.pos, wl.theta, x.wq, x.wk, wl.eps, rope_mode=rope_mode)
    assert_prepass_close(to_host(q), eq, dtype, f"into q D={D} {rope_mode}")
    assert_prepass_close(to_host(k), ek, dtype, f"into k D={D} {rope_mode}")


def test_into_copies_rows_when_nothing_is_requested():
    """No positions and no weights: out of place, the rows are copied exactly
    (in place the same call is a no-op)."""
    import torch
    from vision_encoder_varlen_amd import ops
    wl = W.custom([(9, 11), (3, 5)], H=4, D=80, dtype="bf16", seed=41)
    _, qkv, _, _, _ = _inputs(wl)
    q_src, k_src = qkv[:, 0], qkv[:, 1]
    q, k = torch.zeros_like(q_src.contiguous()), torch.zeros_like(k_src.contiguous())
    ops.qk_norm_rope_into(q_src, k_src, q, k, None)
    torch.cuda.synchronize()
    assert torch.equal(q, q_src) and torch.equal(k, k_src)


def test_into_k_only_and_worklist_in_the_same_launch():
    """k alone (q's half runs inside the attention), with the work-list built
    by the same launch: the list equals the one vit_varlen_worklist builds."""
    import torch
    from vision_encoder_varlen_amd import ops
    wl = W.custom([(6, 8), (17, 5), (32, 32), (1, 1)], H=2, D=128, dtype="bf16", seed=42,
                  use_norm=True)
    x, qkv, pos, _, wk = _inputs(wl)
    before = qkv.clone()
    k_src = qkv[:, 1]
    k = torch.full_like(k_src.contiguous(), float("nan"))
    cu = torch.from_numpy(x.cu_seqlens).cuda()
    bm = ops.attn_block_m(wl.H, wl.D, k.dtype)
    ref = ops.varlen_worklist(cu, wl.max_seqlen, bm)
    plan = ops.varlen_worklist(cu, wl.max_seqlen, bm)
    plan.items.fill_(-7)
    plan.meta.fill_(-7)
    ops.qk_norm_rope_into(None, k_src, None, k, pos, wl.theta, None, wk, wl.eps, plan=plan,
                          cu_seqlens=cu)
    torch.cuda.synchronize()
    assert torch.equal(qkv, before)
    assert torch.equal(plan.meta, ref.meta)
    n = int(ref.meta[0])
    span = min(ref.cap, n + 2048)
    assert torch.equal(plan.items[:span], ref.items[:span])
    _, ek = oracle.qk_norm_rope(x.q, x.k, x.pos, wl.theta, x.wq, x.wk, wl.eps)
    assert_prepass_close(to_host(k), ek, "bf16", "into k only")


def test_into_repeated_calls_give_the_same_rows():
    """Each call starts again from the unchanged sources, so a loop of calls
    (a benchmark's steps) keeps producing the same attention inputs, where the
    in-place call would normalise already normalised rows."""
    import torch
    from vision_encoder_varlen_amd import ops
    wl = W.config(3)
    x, qkv, pos, wq, wk = _inputs(wl)
    q_src, k_src = qkv[:, 0], qkv[:, 1]
    q, k = torch.empty_like(q_src.contiguous()), torch.empty_like(k_src.contiguous())
    ops.qk_norm_rope_into(q_src, k_src, q, k, pos, wl.theta, wq, wk, wl.eps)
    q1, k1 = q.clone(), k.clone()
    for _ in range(5):
        ops.qk_norm_rope_into(q_src, k_src, q, k, pos, wl.theta, wq, wk, wl.eps)
    torch.cuda.synchronize()
    assert torch.equal(q, q1) and torch.equal(k, k1)
    rng = np.random.default_rng(43)
    idx = np.unique(np.concatenate([rng.integers(0, wl.total_tokens, size=1024),
                                    [0, wl.total_tokens - 1]]))
    eq, ek = oracle.qk_norm_rope(x.q[idx], x.k[idx], x.pos[idx], wl.theta, x.wq, x.wk, wl.eps)
    it = torch.from_numpy(idx).cuda()
    assert_prepass_close(to_host(q[it]), eq, "bf16", "repeated into q")
    assert_prepass_close(to_host(k[it]), ek, "bf16", "repeated into k")


def test_into_rejects_overlap_in_python_and_c():
    import torch
    from vision_encoder_varlen_amd import ops, _lib
    wl = W.custom([(4, 4)], H=2, D=64, dtype="bf16", seed=44)
    _, qkv, pos, _, _ = _inputs(wl)
    q_src, k_src = qkv[:, 0], qkv[:, 1]
    k = torch.empty_like(k_src.contiguous())
    # q written over k's source rows
    with pytest.raises(_lib.VitError, match="overlaps"):
        ops.qk_norm_rope_into(q_src, k_src, qkv[:, 2], k, pos)
    with pytest.raises(ValueError):
        ops.qk_norm_rope_into(None, k_src, qkv[:, 2].contiguous(), k, pos)
