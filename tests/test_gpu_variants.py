"""Variants on the pages through the C ABI, against the fp64 oracle:

* the uniform batch (``cu_seqlens = None``): ``vit_dense_batch_attn`` must
  equal the varlen call on ``arange`` boundaries bit for bit, and the oracle
  within the attention tolerance.
"""
import numpy as np
import pytest

import oracle
from vision_encoder_varlen_amd import workloads as W
from gpu_util import assert_attn_close, to_dev, to_host

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


def test_dense_batch_short_segment_workload_sampled():
    """2048 images of 8x8 patches, 16 heads, D = 64 (the many-short-segments
    workload, which is a uniform batch): sampled rows against the oracle."""
    import torch
    from vision_encoder_varlen_amd import ops
    wl = W.config(5)
    x = W.generate(wl)
    q, k, v = (to_dev(a, "bf16") for a in (x.q, x.k, x.v))
    dense = ops.dense_batch_attn(q, k, v, wl.num_seqs, 64)
    cu = torch.from_numpy(x.cu_seqlens).cuda()
    varlen = ops.varlen_attn(q, k, v, cu, wl.max_seqlen)
    torch.cuda.synchronize()
    assert torch.equal(dense, varlen)
    rng = np.random.default_rng(0)
    tok = rng.integers(0, wl.total_tokens, 256)
    hd = rng.integers(0, wl.H, 256)
    want = oracle.varlen_attention_rows(x.q, x.k, x.v, x.cu_seqlens, wl.softmax_scale, tok, hd)
    assert_attn_close(to_host(dense)[tok, hd], want, "bf16", "2048x64 dense batch")


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
