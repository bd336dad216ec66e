"""The whole pre-pass inside the attention kernel
(vit_varlen_attn_planned_qk_norm_rope), through the C ABI.

* q and k in memory are left unchanged;
* the output matches the oracle's end-to-end result (fp64 pre-pass rounded
  once to the storage dtype, then attention) within the attention tolerance,
  for every head dim, both dtypes, both rotary pairings, with and without the
  norm, causal, with the log-sum-exp, on a packed QKV buffer, after the
  exact-max repeat pass, and on empty and one-token segments;
* full-size workloads, every element: the 2048 x 64-token batch (where each
  unit's keys are transformed once, since a segment is one q-tile), the
  ragged batch and the 4 x 1024 batch.
"""
import numpy as np
import pytest

import oracle
from vision_encoder_varlen_amd import workloads as W
from gpu_util import assert_attn_close, to_dev, to_host, workload_oracle

pytestmark = pytest.mark.gpu

GRIDS = [(4, 4), (6, 8), (1, 1), (13, 7), (64, 2), (20, 15)]
LSE_TOL = {"f32": 1e-5, "bf16": 2.0 ** -8}


def _dev_inputs(wl, x):
    import torch
    pos = torch.from_numpy(x.pos).cuda()
    cu = torch.from_numpy(x.cu_seqlens).cuda()
    wq = torch.from_numpy(x.wq).cuda() if wl.use_norm else None
    wk = torch.from_numpy(x.wk).cuda() if wl.use_norm else None
    return pos, cu, wq, wk


def _fused(wl, x, rope_mode="neox", causal=False, with_pos=True):
    """Fused output and the separate pre-pass + attention output, both on the GPU."""
    import torch
    from vision_encoder_varlen_amd import ops
    q, k, v = (to_dev(a, wl.dtype) for a in (x.q, x.k, x.v))
    q0, k0 = q.clone(), k.clone()
    pos, cu, wq, wk = _dev_inputs(wl, x)
    if not with_pos:
        pos = None
    plan = ops.varlen_worklist(cu, wl.max_seqlen, ops.attn_block_m(wl.H, wl.D, q.dtype))
    out = ops.varlen_attn_planned_qk_norm_rope(q, k, v, cu, plan, pos, wl.theta, wq, wk, wl.eps,
                                               rope_mode, causal=causal)
    qr, kr = q.clone(), k.clone()
    ops.qk_norm_rope_(qr, kr, pos, wl.theta, wq, wk, wl.eps, rope_mode=rope_mode)
    ref = ops.varlen_attn_planned(qr, kr, v, cu, plan, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(q, q0) and torch.equal(k, k0), "the fused attention modified q or k"
    return to_host(out), to_host(ref)


def _prepped(wl, x, rope_mode="neox", with_pos=True):
    norm_w = (x.wq, x.wk) if wl.use_norm else (None, None)
    eq, ek = oracle.qk_norm_rope(x.q, x.k, x.pos if with_pos else None, wl.theta, *norm_w,
                                 wl.eps, rope_mode=rope_mode)
    return oracle.round_to_dtype(eq, wl.dtype), oracle.round_to_dtype(ek, wl.dtype)


def _want(wl, x, rope_mode="neox", causal=False, with_pos=True):
    eq, ek = _prepped(wl, x, rope_mode, with_pos)
    return oracle.varlen_attention(eq, ek, x.v, x.cu_seqlens, wl.softmax_scale, causal=causal)


@pytest.mark.parametrize("D", [32, 64, 80, 96, 128])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("norm", [False, True])
@pytest.mark.parametrize("rope_mode", ["neox", "complex"])
def test_fused_qk_matches_oracle(D, dtype, norm, rope_mode):
    wl = W.custom(GRIDS, H=3, D=D, dtype=dtype, seed=120 + D, use_norm=norm)
    x = W.generate(wl)
    got, ref = _fused(wl, x, rope_mode)
    want = _want(wl, x, rope_mode)
    assert_attn_close(got, want, dtype, f"fused qk D={D} {dtype} norm={norm} {rope_mode}")
    assert_attn_close(ref, want, dtype, "separate pre-pass")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_fused_qk_norm_only(dtype):
    """pos = null: the norm alone on both sides."""
    wl = W.custom(GRIDS, H=2, D=80, dtype=dtype, seed=126, use_norm=True)
    x = W.generate(wl)
    got, _ = _fused(wl, x, with_pos=False)
    assert_attn_close(got, _want(wl, x, with_pos=False), dtype, "fused qk norm only")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D", [64, 80, 128])
def test_fused_qk_causal(dtype, D):
    wl = W.custom(GRIDS, H=2, D=D, dtype=dtype, seed=127, use_norm=True)
    x = W.generate(wl)
    got, _ = _fused(wl, x, causal=True)
    assert_attn_close(got, _want(wl, x, causal=True), dtype, "fused qk causal", peaked=True)


def test_fused_qk_large_positions():
    """A 96 x 96 grid (coordinates up to 95), D = 128: several q-tiles per
    segment, each transforming the same K tiles."""
    wl = W.custom([(96, 96)], H=2, D=128, dtype="bf16", seed=128, use_norm=True)
    x = W.generate(wl)
    got, _ = _fused(wl, x)
    assert_attn_close(got, _want(wl, x), "bf16", "fused qk 96x96")


@pytest.mark.parametrize("D", [64, 80, 128])
@pytest.mark.parametrize("rope_mode", ["neox", "complex"])
def test_fused_qk_positions_outside_the_table(D, rope_mode):
    """Negative coordinates and coordinates of 64 and more: the rows and keys
    whose wave has any of them take the directly evaluated angles, the others
    the workgroup's table, in the same launch."""
    wl = W.custom([(10, 13), (7, 9), (3, 40)], H=2, D=D, dtype="bf16", seed=133, use_norm=True)
    x = W.generate(wl)
    rng = np.random.default_rng(133)
    pos = x.pos.astype(np.int64)
    pos[:130] += rng.integers(-200, 200, size=(130, 2))      # first segment: anywhere
    pos[193:] = rng.integers(60, 70, size=(wl.total_tokens - 193, 2))  # straddling 64
    x.pos = pos.astype(np.int32)
    got, _ = _fused(wl, x, rope_mode)
    assert_attn_close(got, _want(wl, x, rope_mode), "bf16", f"fused qk positions D={D}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_fused_qk_empty_and_tiny_segments(dtype):
    """Zero-length, one-token and just-past-a-tile segments (positions (0, l))."""
    wl = W.from_seqlens([0, 1, 0, 33, 65, 2, 0, 129], H=2, D=64, dtype=dtype, seed=129,
                        use_norm=True)
    x = W.generate(wl)
    got, _ = _fused(wl, x, rope_mode="complex")
    assert_attn_close(got, _want(wl, x, rope_mode="complex"), dtype, "fused qk short")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_fused_qk_lse(dtype):
    import torch
    from vision_encoder_varlen_amd import ops
    wl = W.custom(GRIDS, H=3, D=64, dtype=dtype, seed=130, use_norm=True)
    x = W.generate(wl)
    q, k, v = (to_dev(a, dtype) for a in (x.q, x.k, x.v))
    pos, cu, wq, wk = _dev_inputs(wl, x)
    plan = ops.varlen_worklist(cu, wl.max_seqlen, ops.attn_block_m(wl.H, wl.D, q.dtype))
    lse = torch.full((wl.total_tokens, wl.H), float("nan"), dtype=torch.float32, device="cuda")
    out = ops.varlen_attn_planned_qk_norm_rope(q, k, v, cu, plan, pos, wl.theta, wq, wk, wl.eps,
                                               lse=lse)
    plain = ops.varlen_attn_planned_qk_norm_rope(q, k, v, cu, plan, pos, wl.theta, wq, wk, wl.eps)
    torch.cuda.synchronize()
    eq, ek = _prepped(wl, x)
    want = oracle.varlen_lse(eq, ek, x.cu_seqlens, wl.softmax_scale)
    got = lse.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got))
    assert np.max(np.abs(got - want)) <= LSE_TOL[dtype]
    assert torch.equal(out, plain), "the output changed with the log-sum-exp requested"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_fused_qk_packed_qkv_is_bit_identical(dtype):
    """q, k, v as views of one packed [T, 3, H, D] buffer: the same bits as on
    contiguous copies, and the buffer is untouched."""
    import torch
    from vision_encoder_varlen_amd import ops
    wl = W.custom(GRIDS, H=2, D=80, dtype=dtype, seed=131, use_norm=True)
    x = W.generate(wl)
    T, H, D = wl.total_tokens, wl.H, wl.D
    buf = torch.empty((T, 3, H * D), device="cuda",
                      dtype=torch.bfloat16 if dtype == "bf16" else torch.float32)
    for i, a in enumerate((x.q, x.k, x.v)):
        buf[:, i] = to_dev(a, dtype).reshape(T, H * D)
    before = buf.clone()
    q, k, v = (buf[:, i].unflatten(1, (H, D)) for i in range(3))
    pos, cu, wq, wk = _dev_inputs(wl, x)
    plan = ops.varlen_worklist(cu, wl.max_seqlen, ops.attn_block_m(H, D, q.dtype))
    got = ops.varlen_attn_planned_qk_norm_rope(q, k, v, cu, plan, pos, wl.theta, wq, wk, wl.eps)
    ref = ops.varlen_attn_planned_qk_norm_rope(q.contiguous(), k.contiguous(), v.contiguous(),
                                               cu, plan, pos, wl.theta, wq, wk, wl.eps)
    torch.cuda.synchronize()
    assert torch.equal(buf, before), "the packed input was modified"
    assert torch.equal(got, ref)
    assert_attn_close(to_host(got), _want(wl, x), dtype, "fused qk packed")


@pytest.mark.parametrize("D", [64, 80, 128])
def test_fused_qk_repeat_pass(D):
    """Keys after the first key tile score far above every key of that tile
    once normalised (weights 3: logits of about +-9 sqrt(D)), so the exact-max
    repeat pass runs, and it transforms its K tiles again."""
    import torch
    from vision_encoder_varlen_amd.workloads import bf16_bits_to_f32, f32_to_bf16_bits
    lens = [300, 97]
    wl = W.from_seqlens(lens, H=2, D=D, dtype="bf16", seed=132, use_norm=True)
    x = W.generate(wl)
    rng = np.random.default_rng(132)
    u = np.zeros(D, dtype=np.float32)
    u[: D // 2] = 1.0
    q = np.broadcast_to(u, (sum(lens), 2, D)).copy()
    sign = np.where(rng.random((sum(lens), 1, 1)) > 0.5, 1.0, -1.0)
    sign[:64] = -1.0                            # first key tile of each segment: negative
    sign[300:364] = -1.0
    k = sign * u + 0.01 * x.k
    x.q = bf16_bits_to_f32(f32_to_bf16_bits(q.astype(np.float32))).reshape(q.shape)
    x.k = bf16_bits_to_f32(f32_to_bf16_bits(k.astype(np.float32))).reshape(k.shape)
    x.wq = np.full(D, 3.0, dtype=np.float32)
    x.wk = np.full(D, 3.0, dtype=np.float32)
    got, _ = _fused(wl, x, with_pos=False)
    assert_attn_close(got, _want(wl, x, with_pos=False), "bf16", f"fused qk repeat D={D}")
    # the first tile's max really is far below the row max: the repeat ran
    eq, ek = _prepped(wl, x, with_pos=False)
    s = np.einsum("thd,shd->ths", eq[:300], ek[:300]) * wl.softmax_scale
    assert (s.max(axis=2) - s[:, :, :64].max(axis=2)).min() * np.log2(np.e) > 64
    del torch


@pytest.mark.parametrize("n", [2, 3, 5])
def test_fused_qk_workload(n):
    """Full-size workloads, every element against the oracle's end-to-end
    result: 4 x (32 x 32) at D = 80 (rotary only), the 24-image ragged batch
    at D = 128 and 2048 x (8 x 8) at D = 64 (norm and rotary)."""
    import torch
    from vision_encoder_varlen_amd import ops
    wl = W.config(n)
    x = W.generate(wl)
    q, k, v = (to_dev(a, wl.dtype) for a in (x.q, x.k, x.v))
    pos, cu, wq, wk = _dev_inputs(wl, x)
    plan = ops.varlen_worklist(cu, wl.max_seqlen, ops.attn_block_m(wl.H, wl.D, q.dtype))
    out = ops.varlen_attn_planned_qk_norm_rope(q, k, v, cu, plan, pos, wl.theta, wq, wk, wl.eps)
    torch.cuda.synchronize()
    assert_attn_close(to_host(out), workload_oracle(n, "e2e"), wl.dtype, f"config {n} fused qk")
