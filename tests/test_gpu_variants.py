"""Variants on the pages through the C ABI, against the fp64 oracle:

* the uniform batch (``cu_seqlens = None``): ``vit_dense_batch_attn`` must
  equal the varlen call on ``arange`` boundaries bit for bit, and the oracle
  within the attention tolerance;
* the causal flag: the oracle within the attention tolerance (outputs) and
  the log-sum-exp tolerance, every entry point agreeing bit for bit, a
  segment's first row equal to its value row exactly, and the repeat pass
  (a later key far above the first tile) under the causal mask.
"""
import numpy as np
import pytest

import oracle
from vision_encoder_varlen_amd import workloads as W
from gpu_util import assert_attn_close, to_dev, to_host, workload_oracle

pytestmark = pytest.mark.gpu


def _uniform(batch, seq_len, H, D, dtype, seed):
    wl = W.from_seqlens([seq_len] * batch, H=H, D=D, dtype=dtype, seed=seed)
    return wl, W.generate(wl)


@pytest.mark.parametrize("D", [32, 64, 80, 96, 128])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("batch,seq_len", [(3, 200), (5, 64), (2, 1), (1, 300)])
def test_dense_batch_matches_varlen_and_oracle(D, dtype, batch, seq_len):
    import torch
    from vision_encoder_varlen_amd import ops
    wl, x = _uniform(batch, seq_len, 2, D, dtype, seed=D + seq_len)
    q, k, v = (to_dev(a, dtype) for a in (x.q, x.k, x.v))
    cu = torch.from_numpy(oracle.uniform_cu_seqlens(batch, seq_len)).cuda()
    lse_d = torch.empty((batch * seq_len, 2), dtype=torch.float32, device="cuda")
    lse_v = torch.empty_like(lse_d)
    dense = ops.dense_batch_attn(q, k, v, batch, seq_len, lse=lse_d)
    varlen = ops.varlen_attn(q, k, v, cu, seq_len, lse=lse_v)
    torch.cuda.synchronize()
    assert torch.equal(dense, varlen) and torch.equal(lse_d, lse_v)
    want = oracle.dense_batch_attention(x.q, x.k, x.v, batch, seq_len, wl.softmax_scale)
    assert_attn_close(to_host(dense), want, dtype, f"dense batch {batch}x{seq_len} D={D}")


def test_dense_batch_short_segment_workload():
    """2048 images of 8x8 patches, 16 heads, D = 64 (the many-short-segments
    workload, which is a uniform batch): every element against the oracle."""
    import torch
    from vision_encoder_varlen_amd import ops
    wl = W.config(5)
    x = W.generate(wl)
    q, k, v = (to_dev(a, "bf16") for a in (x.q, x.k, x.v))
    dense = torch.full_like(q, float("nan"))
    ops.dense_batch_attn(q, k, v, wl.num_seqs, 64, out=dense)
    cu = torch.from_numpy(x.cu_seqlens).cuda()
    varlen = ops.varlen_attn(q, k, v, cu, wl.max_seqlen)
    torch.cuda.synchronize()
    assert torch.equal(dense, varlen)
    assert_attn_close(to_host(dense), workload_oracle(5, "attn"), "bf16", "2048x64 dense batch")


def test_dense_batch_packed_qkv():
    import torch
    from vision_encoder_varlen_amd import ops
    wl, x = _uniform(4, 130, 3, 80, "bf16", seed=9)
    T = 4 * 130
    qkv = torch.stack([to_dev(a, "bf16") for a in (x.q, x.k, x.v)], dim=1)  # [T, 3, H, D]
    q, k, v = qkv[:, 0], qkv[:, 1], qkv[:, 2]
    got = ops.dense_batch_attn(q, k, v, 4, 130)
    want = ops.dense_batch_attn(q.contiguous(), k.contiguous(), v.contiguous(), 4, 130)
    torch.cuda.synchronize()
    assert torch.equal(got, want) and got.shape == (T, 3, 80)


RAGGED = [1, 7, 64, 65, 127, 128, 129, 300, 700, 0, 2]
LSE_TOL = {"f32": 1e-5, "bf16": 2.0 ** -8}


@pytest.mark.parametrize("D", [32, 64, 80, 96, 128])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_causal_matches_oracle(D, dtype):
    import torch
    from vision_encoder_varlen_amd import ops
    wl = W.from_seqlens(RAGGED, H=3, D=D, dtype=dtype, seed=60 + D)
    x = W.generate(wl)
    q, k, v = (to_dev(a, dtype) for a in (x.q, x.k, x.v))
    cu = torch.from_numpy(x.cu_seqlens).cuda()
    lse = torch.full((wl.total_tokens, 3), float("nan"), dtype=torch.float32, device="cuda")
    out = ops.varlen_attn(q, k, v, cu, wl.max_seqlen, lse=lse, causal=True)
    plain = ops.varlen_attn(q, k, v, cu, wl.max_seqlen, causal=True)
    plan = ops.varlen_worklist(cu, wl.max_seqlen, ops.attn_block_m(3, D, q.dtype))
    planned = ops.varlen_attn_planned(q, k, v, cu, plan, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(out, plain) and torch.equal(out, planned)
    want = oracle.varlen_attention(x.q, x.k, x.v, x.cu_seqlens, wl.softmax_scale, causal=True)
    got = to_host(out)
    assert_attn_close(got, want, dtype, f"causal D={D} {dtype}", peaked=True)
    for a in x.cu_seqlens[:-1]:
        if a < wl.total_tokens:
            assert np.array_equal(got[a], x.v[a].astype(np.float64)), a   # one key, weight 1
    want_lse = oracle.varlen_lse(x.q, x.k, x.cu_seqlens, wl.softmax_scale, causal=True)
    assert np.max(np.abs(lse.cpu().numpy().astype(np.float64) - want_lse)) <= LSE_TOL[dtype]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_causal_dense_batch_equals_varlen(dtype):
    import torch
    from vision_encoder_varlen_amd import ops
    wl, x = _uniform(3, 333, 2, 64, dtype, seed=70)
    q, k, v = (to_dev(a, dtype) for a in (x.q, x.k, x.v))
    cu = torch.from_numpy(oracle.uniform_cu_seqlens(3, 333)).cuda()
    dense = ops.dense_batch_attn(q, k, v, 3, 333, causal=True)
    varlen = ops.varlen_attn(q, k, v, cu, 333, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(dense, varlen)
    want = oracle.dense_batch_attention(x.q, x.k, x.v, 3, 333, wl.softmax_scale, causal=True)
    assert_attn_close(to_host(dense), want, dtype, "causal dense batch", peaked=True)


@pytest.mark.parametrize("D", [80, 128])
def test_causal_logit_jump_forces_repeat(D):
    """Later keys score far above the first key tile, so for rows past them the
    reference max taken from tile 0 must be replaced (the repeat pass); rows
    before the jump never see it."""
    lens = [300, 200]
    wl = W.from_seqlens(lens, H=2, D=D, dtype="bf16", seed=14)
    x = W.generate(wl)
    u = np.zeros(D, dtype=np.float32)
    u[: D // 2] = 1.0
    u /= np.linalg.norm(u)
    big = 4.0 * np.sqrt(D)
    q = np.broadcast_to(big * u, (sum(lens), 2, D)).copy()
    k = x.k.copy() * 0.01
    for a in (0, 300):
        k[a + 150:a + 160] += big * u        # a jump well after the first tile
    from vision_encoder_varlen_amd.workloads import bf16_bits_to_f32, f32_to_bf16_bits
    x.q = bf16_bits_to_f32(f32_to_bf16_bits(q.astype(np.float32))).reshape(q.shape)
    x.k = bf16_bits_to_f32(f32_to_bf16_bits(k.astype(np.float32))).reshape(k.shape)
    import torch
    from vision_encoder_varlen_amd import ops
    qd, kd, vd = (to_dev(a, "bf16") for a in (x.q, x.k, x.v))
    cu = torch.from_numpy(x.cu_seqlens).cuda()
    out = ops.varlen_attn(qd, kd, vd, cu, wl.max_seqlen, causal=True)
    torch.cuda.synchronize()
    want = oracle.varlen_attention(x.q, x.k, x.v, x.cu_seqlens, wl.softmax_scale, causal=True)
    assert_attn_close(to_host(out), want, "bf16", f"causal logit jump D={D}", peaked=True)


def test_causal_ragged_workload():
    """24 images, up to 3100 tokens, D = 128, causal: every element."""
    import torch
    from vision_encoder_varlen_amd import ops
    wl = W.config(3)
    x = W.generate(wl)
    q, k, v = (to_dev(a, "bf16") for a in (x.q, x.k, x.v))
    cu = torch.from_numpy(x.cu_seqlens).cuda()
    out = torch.full_like(q, float("nan"))
    ops.varlen_attn(q, k, v, cu, wl.max_seqlen, causal=True, out=out)
    torch.cuda.synchronize()
    assert_attn_close(to_host(out), workload_oracle(3, "attn", causal=True), "bf16",
                      "ragged24 causal", peaked=True)
