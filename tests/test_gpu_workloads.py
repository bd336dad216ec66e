"""The five seeded workloads at full size, in the launch configuration the
benchmark times: pre-pass then attention through the C ABI, every output
element compared with the oracle.

Two comparisons each:

* attention alone: GPU attention on the seeded q, k, v (no pre-pass) against
  the oracle's attention on the same seeded arrays, so only the attention
  kernel is judged;
* end to end: GPU pre-pass then attention, against the oracle's own fp64
  pre-pass, rounded once to the storage dtype, then its attention.

Every oracle input comes from the seeded generator; none is copied back from
the GPU.  Outputs start as NaN, so a row the kernel never wrote fails.
"""
import numpy as np
import pytest

from vision_encoder_varlen_amd import workloads as W
from gpu_util import assert_attn_close, to_dev, to_host, workload_oracle

pytestmark = pytest.mark.gpu


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


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
def test_workload(n):
    wl = W.config(n)
    x = W.generate(wl)
    print(f"workload {n} ({wl.name}): T={wl.total_tokens} H={wl.H} D={wl.D}", flush=True)
    raw, got = _run_gpu(wl, x)
    assert_attn_close(raw, workload_oracle(n, "attn"), wl.dtype, f"config {n} attention")
    assert_attn_close(got, workload_oracle(n, "e2e"), wl.dtype, f"config {n} end to end")
