"""vit_qk_norm_rope_worklist against the two separate calls: pre-pass results
and work-list bit-identical, through the C ABI."""
import numpy as np
import pytest

from vision_encoder_varlen_amd import workloads as W

pytestmark = pytest.mark.gpu


def _tensors(wl, x):
    import torch
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    dev = torch.device("cuda")
    q, k = (torch.from_numpy(a).to(tdt).to(dev) for a in (x.q, x.k))
    pos = torch.from_numpy(x.pos).to(dev)
    wq = torch.from_numpy(x.wq).to(dev) if wl.use_norm else None
    wk = torch.from_numpy(x.wk).to(dev) if wl.use_norm else None
    cu = torch.from_numpy(x.cu_seqlens).to(dev)
    return q, k, pos, wq, wk, cu


def _compare(wl, x, use_pos=True):
    import torch
    from vision_encoder_varlen_amd import ops
    q, k, pos, wq, wk, cu = _tensors(wl, x)
    if not use_pos:
        pos = None
    bm = ops.attn_block_m(wl.H, wl.D, q.dtype)
    q2, k2 = q.clone(), k.clone()
    ops.qk_norm_rope_(q, k, pos, wl.theta, wq, wk, wl.eps)
    sep = ops.varlen_worklist(cu, wl.max_seqlen, bm)
    fused = ops.varlen_worklist(cu, wl.max_seqlen, bm)
    fused.items.fill_(-7)
    fused.meta.fill_(-7)
    ops.qk_norm_rope_worklist_(q2, k2, pos, wl.theta, wq, wk, wl.eps, fused, cu)
    torch.cuda.synchronize()
    assert torch.equal(q, q2) and torch.equal(k, k2)
    meta_s, meta_f = sep.meta.cpu().numpy(), fused.meta.cpu().numpy()
    assert meta_s[0] == meta_f[0] and meta_s[1] == meta_f[1]
    n = int(meta_s[0])
    span = min(sep.cap, n + 2048)   # the items and the marked rows after them
    assert np.array_equal(sep.items.cpu().numpy()[:span], fused.items.cpu().numpy()[:span])
    return n


@pytest.mark.parametrize("cfg", [1, 2, 3, 5])
def test_fused_equals_separate_on_workload_shapes(cfg):
    wl = W.config(cfg)
    if wl.total_tokens > 40000:      # keep the many-short-segments case small: first 600 images
        wl = W.custom(wl.grids[:600] if wl.grids else [(8, 8)] * 600, H=wl.H, D=wl.D, dtype=wl.dtype,
                      seed=wl.seed, use_norm=wl.use_norm)
    x = W.generate(wl)
    assert _compare(wl, x) > 0


def test_fused_with_large_batch_uses_two_launches():
    # 3000 segments: the list needs more LDS than the pre-pass launch shares.
    wl = W.from_seqlens([1 + (i * 7) % 40 for i in range(3000)], H=2, D=64, dtype="bf16", seed=5,
                        use_norm=True)
    x = W.generate(wl)
    assert _compare(wl, x) == 3000


def test_fused_without_prepass_work_builds_the_list():
    wl = W.from_seqlens([5, 0, 300, 17], H=2, D=32, dtype="bf16", seed=6)
    x = W.generate(wl)
    assert _compare(wl, x, use_pos=False) > 0
