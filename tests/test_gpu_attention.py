"""Attention kernels (bf16 MFMA and fp32) vs the fp64 oracle, plus edge cases
and invariants, all through the C ABI."""
import numpy as np
import pytest

import oracle
from vision_encoder_varlen_amd import workloads as W
from gpu_util import assert_attn_close, to_dev, to_host

pytestmark = pytest.mark.gpu

RAGGED = [1, 7, 64, 65, 127, 128, 129, 300, 700]


def _inputs(lens, H, D, dtype, seed):
    wl = W.from_seqlens(lens, H=H, D=D, dtype=dtype, seed=seed)
    return wl, W.generate(wl)


def _gpu_attn(x, wl, scale=None, max_seqlen=None, guard_rows=0, out_fill=None):
    import torch
    from vision_encoder_varlen_amd import ops
    T = wl.total_tokens
    pad = np.zeros((guard_rows, wl.H, wl.D), dtype=np.float32)
    q = to_dev(np.concatenate([x.q, pad]), wl.dtype)
    k = to_dev(np.concatenate([x.k, pad]), wl.dtype)
    v = to_dev(np.concatenate([x.v, pad]), wl.dtype)
    cu = torch.from_numpy(x.cu_seqlens).cuda()
    out = torch.full_like(q, float("nan") if out_fill is None else out_fill)
    ops.varlen_attn(q, k, v, cu, wl.max_seqlen if max_seqlen is None else max_seqlen,
                    wl.softmax_scale if scale is None else scale, out=out)
    torch.cuda.synchronize()
    got = to_host(out)
    return got[:T], got[T:]


@pytest.mark.parametrize("D", [32, 64, 80, 96, 128])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ragged_layout_matches_oracle(D, dtype):
    wl, x = _inputs(RAGGED, H=3, D=D, dtype=dtype, seed=D)
    got, _ = _gpu_attn(x, wl)
    want = oracle.varlen_attention(x.q, x.k, x.v, x.cu_seqlens, wl.softmax_scale)
    assert_attn_close(got, want, dtype, f"D={D} {dtype}")


@pytest.mark.parametrize("H", [1, 12, 16])
def test_head_counts(H):
    wl, x = _inputs([200, 33, 513], H=H, D=64, dtype="bf16", seed=H)
    got, _ = _gpu_attn(x, wl)
    want = oracle.varlen_attention(x.q, x.k, x.v, x.cu_seqlens, wl.softmax_scale)
    assert_attn_close(got, want, "bf16", f"H={H}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_empty_segments_and_guard_rows(dtype):
    lens = [0, 5, 0, 0, 130, 0, 1]
    wl, x = _inputs(lens, H=2, D=64, dtype=dtype, seed=3)
    got, guard = _gpu_attn(x, wl, guard_rows=16, out_fill=7.0)
    want = oracle.varlen_attention(x.q, x.k, x.v, x.cu_seqlens, wl.softmax_scale)
    assert_attn_close(got, want, dtype, "empty segments")
    assert np.all(guard == 7.0), "rows beyond cu_seqlens[N] were written"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_length_one_segment_returns_its_value_row_bit_exact(dtype):
    wl, x = _inputs([1, 40, 1, 1, 200, 1], H=4, D=128, dtype=dtype, seed=4)
    got, _ = _gpu_attn(x, wl)
    for t in (0, 41, 42, 243):
        assert np.array_equal(got[t], x.v[t].astype(np.float64)), t


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_constant_values_return_the_constant(dtype):
    wl, x = _inputs([77, 300], H=2, D=80, dtype=dtype, seed=5)
    v = x.v.copy()
    v[:77] = v[0]
    v[77:] = v[77]
    x.v = v
    got, _ = _gpu_attn(x, wl)
    tol = 1e-5 if dtype == "f32" else 2.0 ** -7 * np.abs(v).max()
    assert np.max(np.abs(got - v)) <= tol


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_zero_scale_gives_segment_mean(dtype):
    wl, x = _inputs([50, 130], H=2, D=64, dtype=dtype, seed=6)
    got, _ = _gpu_attn(x, wl, scale=0.0)
    want = oracle.varlen_attention(x.q, x.k, x.v, x.cu_seqlens, 0.0)
    assert_attn_close(got, want, dtype, "scale 0")


def test_large_scores_stay_stable():
    wl, x = _inputs([90, 257], H=2, D=128, dtype="bf16", seed=7)
    x.q = x.q * 8.0   # exact in bf16; logits of order 100
    got, _ = _gpu_attn(x, wl)
    want = oracle.varlen_attention(x.q, x.k, x.v, x.cu_seqlens, wl.softmax_scale)
    # Peaked rows return nearly single V rows, some of magnitude 4..8.  There
    # the bf16 weights P (relative rounding 2^-9, as the reference itself
    # rounds P to the input dtype) and the bf16 store of the result (another
    # 2^-9) move an output by up to 2^-8 of its magnitude, which exceeds
    # 1.5e-2 once |out| > 3.8; the bound adds that relative term.
    err = np.abs(got - want)
    tol = 1.5e-2 + 2.0 ** -8 * np.abs(want)
    assert np.all(np.isfinite(got))
    assert np.all(err <= tol), f"peaked softmax: worst {float((err / tol).max()):.3f} of the bound"
    assert np.linalg.norm(got - want) / np.linalg.norm(want) <= 5e-3


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_segment_isolation_is_bit_exact(dtype):
    lens = [100, 260, 31]
    wl, x = _inputs(lens, H=2, D=64, dtype=dtype, seed=8)
    a, _ = _gpu_attn(x, wl)
    for arr in (x.q, x.k, x.v):
        arr[100:360] = arr[100:360] * -0.5
    b, _ = _gpu_attn(x, wl)
    assert np.array_equal(a[:100], b[:100]) and np.array_equal(a[360:], b[360:])
    assert not np.allclose(a[100:360], b[100:360])


def test_segment_permutation_permutes_outputs():
    lens = [100, 260, 31]
    wl, x = _inputs(lens, H=2, D=64, dtype="bf16", seed=9)
    a, _ = _gpu_attn(x, wl)
    cu = x.cu_seqlens
    order = [2, 0, 1]
    idx = np.concatenate([np.arange(cu[i], cu[i + 1]) for i in order])
    wl2 = W.from_seqlens([lens[i] for i in order], H=2, D=64, dtype="bf16")
    x2 = W.Inputs(q=x.q[idx], k=x.k[idx], v=x.v[idx], wq=x.wq, wk=x.wk, pos=x.pos[idx],
                  cu_seqlens=wl2.cu_seqlens)
    b, _ = _gpu_attn(x2, wl2)
    assert np.array_equal(b, a[idx])


def test_results_are_deterministic():
    wl, x = _inputs(RAGGED, H=3, D=80, dtype="bf16", seed=10)
    a, _ = _gpu_attn(x, wl)
    b, _ = _gpu_attn(x, wl)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_planned_path_equals_direct_path(dtype):
    import torch
    from vision_encoder_varlen_amd import ops
    wl, x = _inputs(RAGGED, H=2, D=128, dtype=dtype, seed=11)
    direct, _ = _gpu_attn(x, wl)
    q, k, v = (to_dev(a, dtype) for a in (x.q, x.k, x.v))
    cu = torch.from_numpy(x.cu_seqlens).cuda()
    plan = ops.varlen_worklist(cu, wl.max_seqlen, ops.attn_block_m(2, 128, q.dtype))
    outs = [ops.varlen_attn_planned(q, k, v, cu, plan, wl.softmax_scale) for _ in range(2)]
    torch.cuda.synchronize()
    for o in outs:
        assert np.array_equal(to_host(o), direct)


def test_understated_max_seqlen_skips_and_flags():
    import torch
    from vision_encoder_varlen_amd import ops
    wl, x = _inputs([40, 300, 90], H=2, D=64, dtype="bf16", seed=12)
    ops.device_error(reset=True)
    got, _ = _gpu_attn(x, wl, max_seqlen=128, out_fill=3.0)
    assert ops.device_error() == 4
    assert np.all(got[40:340] == 3.0)
    want = oracle.varlen_attention(x.q, x.k, x.v, x.cu_seqlens, wl.softmax_scale)
    assert_attn_close(got[:40], want[:40], "bf16", "first segment")
    assert_attn_close(got[340:], want[340:], "bf16", "last segment")
    _gpu_attn(x, wl)
    assert ops.device_error() == 0
    torch.cuda.synchronize()


def test_no_segments_is_a_no_op():
    import torch
    from vision_encoder_varlen_amd import ops
    q = torch.zeros((4, 2, 64), dtype=torch.bfloat16, device="cuda")
    out = torch.full_like(q, 5.0)
    ops.varlen_attn(q, q.clone(), q.clone(), torch.zeros(1, dtype=torch.int32, device="cuda"), 0,
                    out=out)
    torch.cuda.synchronize()
    assert torch.all(out == 5.0)


def test_errors_raise_value_error():
    import torch
    from vision_encoder_varlen_amd import ops
    q = torch.zeros((4, 2, 72), dtype=torch.bfloat16, device="cuda")
    cu = torch.tensor([0, 4], dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError, match="head_dim"):
        ops.varlen_attn(q, q.clone(), q.clone(), cu, 4)


@pytest.mark.parametrize("D", [80, 128])
def test_logit_jump_after_first_tile(D):
    """Keys after the first key tile score far above every key of that tile
    (a jump of several hundred logits), so a reference max taken from the first
    tile must be replaced after it was first used."""
    rng = np.random.default_rng(13)
    lens = [300, 97]
    wl = W.from_seqlens(lens, H=2, D=D, dtype="bf16", seed=13)
    x = W.generate(wl)
    u = np.zeros(D, dtype=np.float32)
    u[: D // 2] = 1.0
    u /= np.linalg.norm(u)
    big = 4.0 * np.sqrt(D)                      # |q| = |k| = 4 sqrt(D): logits ~ +-16 D * scale
    q = np.broadcast_to(big * u, (sum(lens), 2, D)).copy()
    k = x.k.copy() * 0.01
    k[:64] -= big * u                          # first 64 keys of each segment: strongly negative
    k[300:364] -= big * u
    jump = rng.random((sum(lens), 1, 1)) > 0.5
    jump[:64] = False
    jump[300:364] = False
    k += big * u * jump                        # about half of the later keys: strongly positive
    x.q = q.astype(np.float32)
    x.k = k.astype(np.float32)
    from vision_encoder_varlen_amd.workloads import bf16_bits_to_f32, f32_to_bf16_bits
    x.q = bf16_bits_to_f32(f32_to_bf16_bits(x.q)).reshape(x.q.shape)
    x.k = bf16_bits_to_f32(f32_to_bf16_bits(x.k)).reshape(x.k.shape)
    got, _ = _gpu_attn(x, wl)
    want = oracle.varlen_attention(x.q, x.k, x.v, x.cu_seqlens, wl.softmax_scale)
    assert_attn_close(got, want, "bf16", f"logit jump D={D}")


SHORT = [1, 2, 31, 32, 33, 0, 63, 64, 17, 48]


@pytest.mark.parametrize("D", [32, 64, 80, 96, 128])
def test_short_segments(D):
    """Many segments shorter than one key tile or one query block."""
    wl, x = _inputs(SHORT, H=4, D=D, dtype="bf16", seed=20 + D)
    got, guard = _gpu_attn(x, wl, guard_rows=8, out_fill=9.0)
    want = oracle.varlen_attention(x.q, x.k, x.v, x.cu_seqlens, wl.softmax_scale)
    assert_attn_close(got, want, "bf16", f"short segments D={D}")
    assert np.all(guard == 9.0)


# Log-sum-exp rows.  fp32: the kernel sums fp32 weights, so 1e-5 absolute (at
# |lse| up to ~10) covers its rounding.  bf16: inputs are exact bf16 values and
# the scores are fp32 MFMA sums; the row sum is of fp32 weights except for head
# dims that are not a multiple of 32, where it comes from the P V MFMA with
# bf16-rounded weights (relative error up to 2^-9 per weight), so the bound is
# 2^-8 absolute on lse.
LSE_TOL = {"f32": 1e-5, "bf16": 2.0 ** -8}


@pytest.mark.parametrize("D", [32, 64, 80, 96, 128])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_lse_matches_oracle(D, dtype):
    import torch
    from vision_encoder_varlen_amd import ops
    wl, x = _inputs(RAGGED + [0, 2], H=3, D=D, dtype=dtype, seed=40 + D)
    q, k, v = (to_dev(a, dtype) for a in (x.q, x.k, x.v))
    cu = torch.from_numpy(x.cu_seqlens).cuda()
    lse = torch.full((wl.total_tokens, 3), float("nan"), dtype=torch.float32, device="cuda")
    out = ops.varlen_attn(q, k, v, cu, wl.max_seqlen, wl.softmax_scale, lse=lse)
    torch.cuda.synchronize()
    want = oracle.varlen_lse(x.q, x.k, x.cu_seqlens, wl.softmax_scale)
    got = lse.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got))
    assert np.max(np.abs(got - want)) <= LSE_TOL[dtype]
    # the output is the same as without lse
    plain, _ = _gpu_attn(x, wl)
    assert np.array_equal(to_host(out), plain)


def test_lse_planned_and_after_a_repeat_pass():
    """Planned call, and a batch whose later keys force the exact-max repeat."""
    import torch
    from vision_encoder_varlen_amd import ops
    D = 128
    lens = [300, 97]
    wl = W.from_seqlens(lens, H=2, D=D, dtype="bf16", seed=13)
    x = W.generate(wl)
    u = np.zeros(D, dtype=np.float32)
    u[: D // 2] = 1.0
    u /= np.linalg.norm(u)
    big = 4.0 * np.sqrt(D)
    x.q = np.broadcast_to(big * u, (sum(lens), 2, D)).astype(np.float32).copy()
    k = x.k * 0.01
    k[:64] -= big * u
    k[300:364] -= big * u
    k[200:210] += big * u
    from vision_encoder_varlen_amd.workloads import bf16_bits_to_f32, f32_to_bf16_bits
    x.q = bf16_bits_to_f32(f32_to_bf16_bits(x.q)).reshape(x.q.shape)
    x.k = bf16_bits_to_f32(f32_to_bf16_bits(k)).reshape(k.shape)
    q, kk, v = (to_dev(a, "bf16") for a in (x.q, x.k, x.v))
    cu = torch.from_numpy(x.cu_seqlens).cuda()
    plan = ops.varlen_worklist(cu, wl.max_seqlen, ops.attn_block_m(2, D, q.dtype))
    lse = torch.empty((sum(lens), 2), dtype=torch.float32, device="cuda")
    ops.varlen_attn_planned(q, kk, v, cu, plan, wl.softmax_scale, lse=lse)
    torch.cuda.synchronize()
    want = oracle.varlen_lse(x.q, x.k, x.cu_seqlens, wl.softmax_scale)
    got = lse.cpu().numpy().astype(np.float64)
    # |lse| is in the hundreds here; fp32 score sums carry ~2^-24 relative error
    assert np.max(np.abs(got - want) / np.maximum(1.0, np.abs(want))) <= 2.0 ** -16
