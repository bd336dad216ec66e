"""vit_varlen_attn_noalloc, the attention entry point that allocates nothing,
against vit_varlen_attn_ex (the allocating call with the same arguments),
through the C ABI.

Two calls in a row, the second with a smaller batch (fewer segments, fewer
work items, another head dim and the causal flag), so the second reads a
work-list that overwrites a longer one in the same fixed device array.  Each
call must equal the allocating call bit for bit (out and lse) and be within
the attention tolerance of the oracle.
"""
import numpy as np
import pytest

import oracle
from vision_encoder_varlen_amd import _lib
from vision_encoder_varlen_amd import workloads as W
from gpu_util import assert_attn_close, to_dev, to_host

pytestmark = pytest.mark.gpu

LSE_TOL = {"f32": 1e-5, "bf16": 2.0 ** -8}


def _lengths(seed, n, hi):
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, hi, size=n)
    lens[::11] = 0
    return [int(x) for x in lens]


def _run(fn, wl, x, flags):
    import torch
    q, k, v = (to_dev(a, wl.dtype) for a in (x.q, x.k, x.v))
    cu = torch.from_numpy(x.cu_seqlens).cuda()
    out = torch.full_like(q, float("nan"))
    lse = torch.full((wl.total_tokens, wl.H), float("nan"), dtype=torch.float32, device="cuda")
    dcode = _lib.VIT_BF16 if wl.dtype == "bf16" else _lib.VIT_F32
    stream = torch.cuda.current_stream().cuda_stream
    _lib.check(fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), cu.data_ptr(), wl.num_seqs,
                  wl.max_seqlen, wl.H, wl.D, float(wl.softmax_scale), dcode, flags,
                  out.data_ptr(), lse.data_ptr(), None, stream))
    return out, lse


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_matches_allocating_call(dtype):
    import torch
    lib = _lib.load()
    calls = [  # (lengths, H, D, flags): the second is smaller than the first
        (_lengths(1, 300, 400), 8, 80, 0),
        (_lengths(2, 9, 200), 2, 128, _lib.VIT_ATTN_CAUSAL),
    ]
    for i, (lens, H, D, flags) in enumerate(calls):
        wl = W.from_seqlens(lens, H=H, D=D, dtype=dtype, seed=500 + i)
        x = W.generate(wl)
        print(f"call {i}: {dtype} {wl.num_seqs} segments, {wl.total_tokens} tokens, H={H} D={D} "
              f"flags={flags}", flush=True)
        out_n, lse_n = _run(lib.vit_varlen_attn_noalloc, wl, x, flags)
        out_e, lse_e = _run(lib.vit_varlen_attn_ex, wl, x, flags)
        torch.cuda.synchronize()
        assert torch.equal(out_n, out_e), f"call {i}: out differs from vit_varlen_attn_ex"
        assert torch.equal(lse_n, lse_e), f"call {i}: lse differs from vit_varlen_attn_ex"
        causal = bool(flags & _lib.VIT_ATTN_CAUSAL)
        want = oracle.varlen_attention(x.q, x.k, x.v, x.cu_seqlens, wl.softmax_scale, causal=causal)
        assert_attn_close(to_host(out_n), want, dtype, f"no-alloc call {i}", peaked=causal)
        want_lse = oracle.varlen_lse(x.q, x.k, x.cu_seqlens, wl.softmax_scale, causal=causal)
        err = np.max(np.abs(lse_n.cpu().numpy().astype(np.float64) - want_lse))
        assert err <= LSE_TOL[dtype], f"call {i}: lse error {err}"
