"""The five seeded workloads at full size, in the launch configuration the
benchmark times: pre-pass then attention through the C ABI.

Small workloads (65 and 4096 tokens) are compared element by element with the
oracle.  The large ones are compared on sampled output rows, each computed by
the oracle on its own, plus properties that hold at any size (every row finite
and written, nothing outside the batch touched).  Two comparisons each:

* attention alone: GPU attention on the seeded q, k, v (no pre-pass) against
  the oracle's attention on the same seeded arrays, so only the attention
  kernel is judged;
* end to end: GPU pre-pass then attention, against the oracle's own fp64
  pre-pass, rounded once to the storage dtype, then its attention.
Every oracle input comes from the seeded generator; none is copied back from
the GPU.
"""
import numpy as np
import pytest

import oracle
from vision_encoder_varlen_amd import workloads as W
from gpu_util import assert_attn_close, to_dev, to_host

pytestmark = pytest.mark.gpu

FULL = {1, 2}
SAMPLE_ROWS = 768


def _run_gpu(wl, x):
    """(attention on the seeded inputs, pre-pass + attention), both on the host."""
    import torch
    from vision_encoder_varlen_amd import ops
    q, k, v = (to_dev(a, wl.dtype) for a in (x.q, x.k, x.v))
    pos = torch.from_numpy(x.pos).cuda()
    cu = torch.from_numpy(x.cu_seqlens).cuda()
    wq = torch.from_numpy(x.wq).cuda() if wl.use_norm else None
    wk = torch.from_numpy(x.wk).cuda() if wl.use_norm else None
    raw = torch.full_like(q, float("nan"))
    ops.varlen_attn(q, k, v, cu, wl.max_seqlen, wl.softmax_scale, out=raw)
    out = torch.full_like(q, float("nan"))
    ops.qk_norm_rope_(q, k, pos, wl.theta, wq, wk, wl.eps)
    ops.varlen_attn(q, k, v, cu, wl.max_seqlen, wl.softmax_scale, out=out)
    torch.cuda.synchronize()
    assert ops.device_error() == 0
    return to_host(raw), to_host(out)


def _sample(wl, rng):
    tok = rng.integers(0, wl.total_tokens, size=SAMPLE_ROWS)
    cu = wl.cu_seqlens
    # always include first and last rows of the first and last segments
    extra = [0, int(cu[1]) - 1, int(cu[-2]), wl.total_tokens - 1]
    tok = np.concatenate([tok, extra])
    heads = rng.integers(0, wl.H, size=tok.shape[0])
    return tok, heads


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
def test_workload(n):
    import torch
    wl = W.config(n)
    x = W.generate(wl)
    raw, got = _run_gpu(wl, x)
    assert np.all(np.isfinite(got)) and np.all(np.isfinite(raw)), "some output row was not written"
    scale = wl.softmax_scale
    norm_w = (x.wq, x.wk) if wl.use_norm else (None, None)

    if n in FULL:
        # attention alone, on the seeded inputs
        want = oracle.varlen_attention(x.q, x.k, x.v, x.cu_seqlens, scale)
        assert_attn_close(raw, want, wl.dtype, f"config {n} attention")
        # end to end
        eq, ek = oracle.qk_norm_rope(x.q, x.k, x.pos, wl.theta, *norm_w, wl.eps)
        eq, ek = oracle.round_to_dtype(eq, wl.dtype), oracle.round_to_dtype(ek, wl.dtype)
        want_e2e = oracle.varlen_attention(eq, ek, x.v, x.cu_seqlens, scale)
        assert_attn_close(got, want_e2e, wl.dtype, f"config {n} end to end")
        return

    rng = np.random.default_rng(500 + n)
    tok, heads = _sample(wl, rng)
    cu = x.cu_seqlens
    seg = np.searchsorted(cu, tok, side="right") - 1
    segs = np.unique(seg)
    idx = np.concatenate([np.arange(cu[s], cu[s + 1]) for s in segs])
    # attention alone, on the seeded inputs
    want = oracle.varlen_attention_rows(x.q, x.k, x.v, cu, scale, tok, heads)
    assert_attn_close(raw[tok, heads], want, wl.dtype, f"config {n} attention (sampled)")
    # end to end on the same sample (the oracle pre-pass on the touched segments)
    eq = np.zeros(x.q.shape, dtype=np.float64)
    ek = np.zeros(x.k.shape, dtype=np.float64)
    pq, pk = oracle.qk_norm_rope(x.q[idx], x.k[idx], x.pos[idx], wl.theta, *norm_w, wl.eps)
    eq[idx] = oracle.round_to_dtype(pq, wl.dtype)
    ek[idx] = oracle.round_to_dtype(pk, wl.dtype)
    want_e2e = oracle.varlen_attention_rows(eq, ek, x.v, cu, scale, tok, heads)
    assert_attn_close(got[tok, heads], want_e2e, wl.dtype, f"config {n} end to end (sampled)")
