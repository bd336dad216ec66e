"""Token-strided inputs and outputs through the C ABI: views of a packed
[T, 3, H, D] QKV projection, and an output buffer wider than H * D.  Each
result must be bit-identical to the same call on contiguous copies (the kernels
do the same arithmetic; only the addressing differs), and nothing outside the
viewed elements may be written."""
import numpy as np
import pytest

import oracle
from vision_encoder_varlen_amd import workloads as W
from gpu_util import assert_attn_close, to_dev, to_host

pytestmark = pytest.mark.gpu

RAGGED = [1, 7, 64, 65, 127, 128, 129, 300, 700]


def _packed(x, wl, pad_cols=0):
    """q, k, v as views of one [T, 3, H*D + pad] buffer (token stride 3*(H*D + pad))."""
    import torch
    T, H, D = wl.total_tokens, wl.H, wl.D
    buf = torch.full((T, 3, H * D + pad_cols), 5.0, device="cuda",
                     dtype=torch.bfloat16 if wl.dtype == "bf16" else torch.float32)
    for i, a in enumerate((x.q, x.k, x.v)):
        buf[:, i, :H * D] = to_dev(a, wl.dtype).reshape(T, H * D)
    views = [buf[:, i, :H * D].unflatten(1, (H, D)) for i in range(3)]
    return buf, views


def _wide_out(wl, pad_cols):
    import torch
    T, H, D = wl.total_tokens, wl.H, wl.D
    wide = torch.full((T, H * D + pad_cols), 9.0, device="cuda",
                      dtype=torch.bfloat16 if wl.dtype == "bf16" else torch.float32)
    return wide, wide[:, :H * D].unflatten(1, (H, D))


@pytest.mark.parametrize("D", [64, 80, 128])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("pad_cols", [0, 64])
def test_packed_qkv_attention_is_bit_identical(D, dtype, pad_cols):
    import torch
    from vision_encoder_varlen_amd import ops
    wl = W.from_seqlens(RAGGED, H=3, D=D, dtype=dtype, seed=11 + D)
    x = W.generate(wl)
    buf, (q, k, v) = _packed(x, wl, pad_cols)
    assert q.stride(0) == 3 * (wl.H * D + pad_cols) and not q.is_contiguous()
    cu = torch.from_numpy(x.cu_seqlens).cuda()
    dense = ops.varlen_attn(q.contiguous(), k.contiguous(), v.contiguous(), cu, wl.max_seqlen)
    wide, out = _wide_out(wl, 32)
    before = buf.clone()
    ops.varlen_attn(q, k, v, cu, wl.max_seqlen, out=out)
    torch.cuda.synchronize()
    assert torch.equal(out, dense), "strided result differs from the contiguous one"
    assert torch.all(wide[:, wl.H * D:] == 9.0), "output padding columns were written"
    assert torch.equal(buf, before), "the packed input was modified"
    want = oracle.varlen_attention(x.q, x.k, x.v, x.cu_seqlens, wl.softmax_scale)
    assert_attn_close(to_host(out), want, dtype, f"packed D={D} {dtype}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_packed_qkv_lse_and_planned_path(dtype):
    import torch
    from vision_encoder_varlen_amd import ops
    wl = W.from_seqlens([513, 0, 40, 1024, 3], H=4, D=80, dtype=dtype, seed=21)
    x = W.generate(wl)
    _, (q, k, v) = _packed(x, wl)
    cu = torch.from_numpy(x.cu_seqlens).cuda()
    T, H = wl.total_tokens, wl.H
    lse_d = torch.empty((T, H), dtype=torch.float32, device="cuda")
    dense = ops.varlen_attn(q.contiguous(), k.contiguous(), v.contiguous(), cu, wl.max_seqlen,
                            lse=lse_d)
    lse_s = torch.full((T, H), 3.0, dtype=torch.float32, device="cuda")
    got = ops.varlen_attn(q, k, v, cu, wl.max_seqlen, lse=lse_s)
    plan = ops.varlen_worklist(cu, wl.max_seqlen, ops.attn_block_m(H, wl.D, q.dtype))
    wide, out_p = _wide_out(wl, 16)
    lse_p = torch.empty_like(lse_s)
    ops.varlen_attn_planned(q, k, v, cu, plan, out=out_p, lse=lse_p)
    torch.cuda.synchronize()
    assert torch.equal(got, dense) and torch.equal(lse_s, lse_d)
    assert torch.equal(out_p, dense) and torch.equal(lse_p, lse_d)
    assert torch.all(wide[:, H * wl.D:] == 9.0)
    want = oracle.varlen_lse(x.q, x.k, x.cu_seqlens, wl.softmax_scale)
    tol = 1e-5 if dtype == "f32" else 2.0 ** -8
    err = np.abs(lse_s.cpu().numpy().astype(np.float64) - want)
    assert err.max() <= tol, err.max()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_packed_prepass_is_bit_identical_and_leaves_v_alone(dtype):
    import torch
    from vision_encoder_varlen_amd import ops
    wl = W.custom([(6, 8), (17, 5), (32, 32)], H=3, D=64, dtype=dtype, seed=7, use_norm=True)
    x = W.generate(wl)
    buf, (q, k, v) = _packed(x, wl)
    qd, kd = q.contiguous(), k.contiguous()
    v_before = v.clone()
    pos = torch.from_numpy(x.pos).cuda()
    wq, wk = torch.from_numpy(x.wq).cuda(), torch.from_numpy(x.wk).cuda()
    ops.qk_norm_rope_(qd, kd, pos, wl.theta, wq, wk, wl.eps)
    ops.qk_norm_rope_(q, k, pos, wl.theta, wq, wk, wl.eps)
    torch.cuda.synchronize()
    assert torch.equal(q, qd) and torch.equal(k, kd)
    assert torch.equal(v, v_before), "the pre-pass wrote into v"


def test_packed_fused_prepass_worklist():
    import torch
    from vision_encoder_varlen_amd import ops
    wl = W.custom([(6, 8), (17, 5), (32, 32), (1, 1)], H=2, D=80, dtype="bf16", seed=8,
                  use_norm=True)
    x = W.generate(wl)
    _, (q, k, v) = _packed(x, wl)
    qd, kd = q.contiguous(), k.contiguous()
    pos = torch.from_numpy(x.pos).cuda()
    wq, wk = torch.from_numpy(x.wq).cuda(), torch.from_numpy(x.wk).cuda()
    cu = torch.from_numpy(x.cu_seqlens).cuda()
    bm = ops.attn_block_m(wl.H, wl.D, q.dtype)
    sep = ops.varlen_worklist(cu, wl.max_seqlen, bm)
    ops.qk_norm_rope_(qd, kd, pos, wl.theta, wq, wk, wl.eps)
    fused = ops.varlen_worklist(cu, wl.max_seqlen, bm)
    fused.meta.fill_(-7)
    ops.qk_norm_rope_worklist_(q, k, pos, wl.theta, wq, wk, wl.eps, fused, cu)
    out = ops.varlen_attn_planned(q, k, v, cu, fused)
    dense = ops.varlen_attn_planned(qd, kd, v.contiguous(), cu, sep)
    torch.cuda.synchronize()
    assert torch.equal(q, qd) and torch.equal(k, kd)
    assert torch.equal(fused.meta, sep.meta)
    assert torch.equal(out, dense)
