"""Seeded combinations of the attention options through the C ABI, against
the fp64 oracle: ragged lengths (zero-length and single-token segments
included), head counts, head dims, both dtypes, the causal flag, the
log-sum-exp output, packed [T, 3, H, D] input views and a wider output buffer,
on both the direct and the planned entry points.  Each case is drawn from its
own seed, so a failure names its case."""
import numpy as np
import pytest

import oracle
from vision_encoder_varlen_amd import workloads as W
from gpu_util import assert_attn_close, to_dev, to_host

pytestmark = pytest.mark.gpu

LSE_TOL = {"f32": 1e-5, "bf16": 2.0 ** -8}
N_CASES = 24


def _case(i):
    rng = np.random.default_rng(1000 + i)
    n = int(rng.integers(1, 9))
    lens = [int(v) for v in rng.choice([0, 1, 2, 31, 64, 127, 128, 129, 300, 777], size=n)]
    if sum(lens) == 0:
        lens[0] = 5
    return dict(lens=lens,
                H=int(rng.integers(1, 7)),
                D=int(rng.choice([32, 64, 80, 96, 128])),
                dtype=str(rng.choice(["bf16", "f32"])),
                causal=bool(rng.integers(0, 2)),
                lse=bool(rng.integers(0, 2)),
                packed=bool(rng.integers(0, 2)),
                planned=bool(rng.integers(0, 2)),
                seed=2000 + i)


@pytest.mark.parametrize("i", range(N_CASES))
def test_option_combinations(i):
    import torch
    from vision_encoder_varlen_amd import ops
    c = _case(i)
    wl = W.from_seqlens(c["lens"], H=c["H"], D=c["D"], dtype=c["dtype"], seed=c["seed"])
    x = W.generate(wl)
    T, H, D = wl.total_tokens, wl.H, wl.D
    if c["packed"]:
        qkv = torch.stack([to_dev(a, c["dtype"]) for a in (x.q, x.k, x.v)], dim=1)
        q, k, v = qkv[:, 0], qkv[:, 1], qkv[:, 2]
        wide = torch.full((T, H * D + 16), 7.0, dtype=q.dtype, device="cuda")
        out = wide[:, :H * D].unflatten(1, (H, D))
    else:
        q, k, v = (to_dev(a, c["dtype"]) for a in (x.q, x.k, x.v))
        wide = None
        out = torch.full_like(q, float("nan"))
    cu = torch.from_numpy(x.cu_seqlens).cuda()
    lse = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda") if c["lse"] else None
    if c["planned"]:
        plan = ops.varlen_worklist(cu, wl.max_seqlen, ops.attn_block_m(H, D, q.dtype))
        ops.varlen_attn_planned(q, k, v, cu, plan, out=out, lse=lse, causal=c["causal"])
    else:
        ops.varlen_attn(q, k, v, cu, wl.max_seqlen, out=out, lse=lse, causal=c["causal"])
    torch.cuda.synchronize()
    what = f"case {i}: {c}"
    want = oracle.varlen_attention(x.q, x.k, x.v, x.cu_seqlens, wl.softmax_scale, causal=c["causal"])
    assert_attn_close(to_host(out), want, c["dtype"], what, peaked=c["causal"])
    if wide is not None:
        assert torch.all(wide[:, H * D:] == 7.0), what
    if lse is not None:
        want_lse = oracle.varlen_lse(x.q, x.k, x.cu_seqlens, wl.softmax_scale, causal=c["causal"])
        err = np.abs(lse.cpu().numpy().astype(np.float64) - want_lse)
        assert np.max(err) <= LSE_TOL[c["dtype"]], what
