"""More work units than the bf16 kernel's grid, every element against the oracle.

The bf16 attention grid is capped at 2048 workgroups; beyond that each
workgroup loops over several (segment, q-tile, head) units, reusing its LDS
ring and its copy offsets, and letting a unit's output stores drain under the
next unit's loads.  These batches have
several thousand units of mixed kinds (multi-tile segments, ragged last tiles,
64-key single tiles, empty segments) so that every workgroup runs two or more
of them, through each entry point that launches the kernel: the plain call,
the causal flag, the log-sum-exp output, the planned call and the planned
call with q's norm and rotary inside the kernel.
"""
import numpy as np
import pytest

import oracle
from vision_encoder_varlen_amd import workloads as W
from gpu_util import assert_attn_close, to_dev, to_host

pytestmark = pytest.mark.gpu

GRID_CAP = 2048
LSE_TOL_BF16 = 2.0 ** -8


def _lengths(seed, n=320):
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, 400, size=n)
    lens[::37] = 0                      # some empty segments
    lens[5::41] = 64                    # exactly one key tile
    return [int(x) for x in lens]


def _bm(H, D):
    import torch
    from vision_encoder_varlen_amd import ops
    return ops.attn_block_m(H, D, torch.bfloat16)


def _units(lens, H, D):
    bm = _bm(H, D)
    return sum((n + bm - 1) // bm for n in lens) * H


@pytest.mark.parametrize("D", [64, 80, 128])
def test_multi_unit_workgroups(D):
    import torch
    from vision_encoder_varlen_amd import ops
    H = 8
    lens = _lengths(100 + D, n=320 * _bm(H, D) // 128)  # more segments for taller q-tiles
    assert _units(lens, H, D) > 2 * GRID_CAP
    wl = W.from_seqlens(lens, H=H, D=D, dtype="bf16", seed=200 + D)
    x = W.generate(wl)
    print(f"D={D}: {wl.num_seqs} segments, {wl.total_tokens} tokens, {_units(lens, H, D)} units",
          flush=True)
    q, k, v = (to_dev(a, "bf16") for a in (x.q, x.k, x.v))
    cu = torch.from_numpy(x.cu_seqlens).cuda()
    nan = lambda: torch.full_like(q, float("nan"))  # noqa: E731
    out, out_c, out_p = nan(), nan(), nan()
    lse = torch.full((wl.total_tokens, H), float("nan"), dtype=torch.float32, device="cuda")
    ops.varlen_attn(q, k, v, cu, wl.max_seqlen, out=out)
    with_lse = ops.varlen_attn(q, k, v, cu, wl.max_seqlen, lse=lse)
    ops.varlen_attn(q, k, v, cu, wl.max_seqlen, causal=True, out=out_c)
    plan = ops.varlen_worklist(cu, wl.max_seqlen, ops.attn_block_m(H, D, q.dtype))
    ops.varlen_attn_planned(q, k, v, cu, plan, out=out_p)
    torch.cuda.synchronize()
    assert ops.device_error() == 0
    assert torch.equal(out, with_lse) and torch.equal(out, out_p)

    want = oracle.varlen_attention(x.q, x.k, x.v, x.cu_seqlens, wl.softmax_scale)
    assert_attn_close(to_host(out), want, "bf16", f"multi-unit D={D}")
    want_lse = oracle.varlen_lse(x.q, x.k, x.cu_seqlens, wl.softmax_scale)
    lse_err = np.max(np.abs(lse.cpu().numpy().astype(np.float64) - want_lse))
    assert lse_err <= LSE_TOL_BF16, f"lse error {lse_err}"
    want_c = oracle.varlen_attention(x.q, x.k, x.v, x.cu_seqlens, wl.softmax_scale, causal=True)
    assert_attn_close(to_host(out_c), want_c, "bf16", f"multi-unit causal D={D}", peaked=True)


@pytest.mark.parametrize("D", [80, 128])
def test_multi_unit_workgroups_fused_q(D):
    """The planned call with q's norm and rotary inside the kernel: each unit
    normalises and rotates its Q fragments in registers while its first K/V
    tiles are in flight behind the previous unit's stores."""
    import torch
    from vision_encoder_varlen_amd import ops
    H = 8
    lens = _lengths(300 + D, n=320 * _bm(H, D) // 128)
    # grids for the rotary positions: an h x w image per segment needs h * w
    # tokens, so take each length's widest factorisation (1 x n for primes)
    grids = []
    for n in lens:
        h = max(f for f in range(1, int(np.sqrt(max(n, 1))) + 1) if n % f == 0) if n else 0
        grids.append((h, n // h) if n else (0, 0))
    wl = W.custom(grids, H=H, D=D, dtype="bf16", seed=400 + D, use_norm=True)
    x = W.generate(wl)
    assert list(np.diff(x.cu_seqlens)) == lens
    assert _units(lens, H, D) > 2 * GRID_CAP
    q, k, v = (to_dev(a, "bf16") for a in (x.q, x.k, x.v))
    pos = torch.from_numpy(x.pos).cuda()
    cu = torch.from_numpy(x.cu_seqlens).cuda()
    wq = torch.from_numpy(x.wq).cuda()
    wk = torch.from_numpy(x.wk).cuda()
    ops.qk_norm_rope_(None, k, pos, wl.theta, None, wk, wl.eps)
    plan = ops.varlen_worklist(cu, wl.max_seqlen, ops.attn_block_m(H, D, q.dtype))
    out = torch.full_like(q, float("nan"))
    ops.varlen_attn_planned_qnorm_rope(q, k, v, cu, plan, pos, wl.theta, wq, wl.eps, out=out)
    torch.cuda.synchronize()
    eq, ek = oracle.qk_norm_rope(x.q, x.k, x.pos, wl.theta, x.wq, x.wk, wl.eps)
    eq, ek = oracle.round_to_bf16(eq), oracle.round_to_bf16(ek)
    want = oracle.varlen_attention(eq, ek, x.v, x.cu_seqlens, wl.softmax_scale)
    assert_attn_close(to_host(out), want, "bf16", f"multi-unit fused q D={D}")


@pytest.mark.parametrize("H,D", [(12, 64), (6, 128), (3, 80)])
def test_multi_unit_head_major_order(H, D):
    """Head counts that are not a multiple of 8 take the units head-major, in
    one contiguous chunk per XCD, reading the list length; more units than
    the grid, so each workgroup runs several, through the list (plain and
    causal) and the uniform batch."""
    import torch
    from vision_encoder_varlen_amd import ops
    lens = _lengths(700 + H, n=48 * 8 // H * 8 * _bm(H, D) // 128)
    wl = W.from_seqlens(lens, H=H, D=D, dtype="bf16", seed=800 + H)
    x = W.generate(wl)
    assert _units(lens, H, D) > 2 * GRID_CAP
    q, k, v = (to_dev(a, "bf16") for a in (x.q, x.k, x.v))
    cu = torch.from_numpy(x.cu_seqlens).cuda()
    out, out_c = torch.full_like(q, float("nan")), torch.full_like(q, float("nan"))
    ops.varlen_attn(q, k, v, cu, wl.max_seqlen, out=out)
    ops.varlen_attn(q, k, v, cu, wl.max_seqlen, causal=True, out=out_c)
    torch.cuda.synchronize()
    want = oracle.varlen_attention(x.q, x.k, x.v, x.cu_seqlens, wl.softmax_scale)
    assert_attn_close(to_host(out), want, "bf16", f"head-major H={H} D={D}")
    want_c = oracle.varlen_attention(x.q, x.k, x.v, x.cu_seqlens, wl.softmax_scale, causal=True)
    assert_attn_close(to_host(out_c), want_c, "bf16", f"head-major causal H={H} D={D}",
                      peaked=True)
    # uniform batch: 600 segments of 100 tokens
    wu = W.from_seqlens([100] * 600, H=H, D=D, dtype="bf16", seed=900 + H)
    xu = W.generate(wu)
    qu, ku, vu = (to_dev(a, "bf16") for a in (xu.q, xu.k, xu.v))
    dense = torch.full_like(qu, float("nan"))
    ops.dense_batch_attn(qu, ku, vu, 600, 100, out=dense)
    torch.cuda.synchronize()
    want_u = oracle.dense_batch_attention(xu.q, xu.k, xu.v, 600, 100, wu.softmax_scale)
    assert_attn_close(to_host(dense), want_u, "bf16", f"head-major uniform H={H} D={D}")
