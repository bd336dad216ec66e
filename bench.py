"""Benchmark: one step = the whole hot path on one packed batch.

Step = Q/K RMSNorm + 2D RoPE pre-pass and work-list build (one launch,
vit_qk_norm_rope_into: from the projection's q and k, which stay unchanged,
into the attention's q and k), then varlen attention (vit_varlen_attn_planned)
-- enqueued on the current stream through the C ABI, with inputs resident in
HBM before timing starts.  Every step thus normalises the same rows; a pre-pass
in place would normalise its own output again each step, and repeated RMSNorm
with unequal weights drives the rows towards their largest-weight channels
(near-zero MFMA operands, which run faster than real data).

Default workload: 4 images of 32x32 patches (4096 tokens), 16 heads, head dim
80, bf16, RoPE only (the workload the attention metric is quoted on).  The
metric is attention TFLOP/s with FLOPs = 4*H*D*sum(s_i^2) per step.

The attention kernel's own average duration is measured live inside the timed
loop with HIP events that the kernel's dispatch records at its start and end
(hipExtLaunchKernel, on the stream it is launched on); the roofline fraction is
taken against MI355X's dense bf16 MFMA peak.  With the default workload the
line also carries the attention kernel alone on the ragged 24-image batch
(second_target), the other workload the 50%-of-peak target is set on.

Before the W warm-up steps the step runs untimed for at least --settle-ms
(default 1 s, reported under "settle"): the chip's clock climbs for a few
hundred milliseconds of sustained load, and the timed steps are meant to run at
the clock it holds in continuous use.

Memory-bound side timings (the pre-pass, and the attention once more) read a
1 GiB buffer before each launch, so their inputs come from HBM rather than
from the Infinity Cache.  Kernel durations are reported as mean and median.
The CPU oracle is timed on a bounded sample of the same workload on the host
cores, with the BLAS library it runs on and its wall-seconds on every seeded
workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config N]
                       [--no-cpu-baseline] [--traffic-json FILE]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "varlen ViT attention TFLOP/s (4·H·D·Σsᵢ²) and % of MI355X bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_F32_VALU_TFLOPS = 157.3  # MI355X fp32 vector
PEAK_HBM_GBPS = 8000.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=400,
                   help="timed steps (the attention is sampled on every --hook-every-th: 50 samples)")
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--config", type=int, default=2, help="seeded workload 1..5 (default 2)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--hook-every", type=int, default=8,
                   help="time the attention kernel on every N-th step of the timed loop")
    p.add_argument("--causal", action="store_true",
                   help="causal variant (query a sees keys 0..a of its segment); FLOPs count "
                        "the unmasked pairs, 4*H*D*sum(s*(s+1)/2)")
    p.add_argument("--fuse-q", action="store_true",
                   help="q's RMSNorm + rotary inside the attention kernel; the pre-pass "
                        "launch handles k only")
    p.add_argument("--fuse-qk", action="store_true",
                   help="the whole pre-pass (q and k) inside the attention kernel; the step's "
                        "first launch only builds the work-list")
    p.add_argument("--dense-batch", action="store_true",
                   help="uniform workloads only: attention through vit_dense_batch_attn "
                        "(cu_seqlens = None form: no work-list, no metadata reads)")
    p.add_argument("--packed-qkv", action="store_true",
                   help="read q, k, v as views of one packed [T, 3, H, D] buffer (token stride 3*H*D)")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="approximate CPU-oracle time budget")
    p.add_argument("--no-oracle-per-config", action="store_true",
                   help="skip the oracle's wall-seconds on every seeded workload in cpu_baseline")
    p.add_argument("--second-target", type=int, default=3, metavar="N",
                   help="with the default workload (2): also time the attention kernel alone on "
                        "seeded workload N (default 3, the ragged batch; 0 = off) and report it "
                        "under second_target")
    p.add_argument("--settle-ms", type=float, default=1000.0,
                   help="untimed steps for at least this many milliseconds before the warm-up "
                        "steps (and before the second target's launches): the chip raises its "
                        "clock over the first few hundred ms of sustained load, and the timed "
                        "steps should run at the clock it then holds")
    p.add_argument("--flush-mib", type=int, default=1024,
                   help="size of the buffer read before each memory-bound side-loop launch, "
                        "so its inputs come from HBM and not the 256 MB Infinity Cache")
    p.add_argument("--traffic-json", default="",
                   help="HBM traffic per attention launch measured by rocprofv3 counters "
                        "(default profiles/attn_traffic_<workload>.json)")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="run one device-to-device copy of MIB MiB before warm-up, as the known-size "
                        "kernel that scales rocprofv3's FETCH_SIZE / WRITE_SIZE counters")
    p.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                   help="no GPU: turn the counter_collection.csv files of a FETCH_SIZE pass and a "
                        "WRITE_SIZE pass (over a run with --copy-calibration) into --traffic-json")
    p.add_argument("--calibration-meta", default="", metavar="JSON",
                   help="with --copy-calibration: where to write the copy size and workload; "
                        "with --summarize-pmc: where to read them")
    p.add_argument("--pmc-command", default="",
                   help="with --summarize-pmc: the profiling command, stored with the result")
    return p.parse_args()


def _counter_rows(path, counter):
    """(kernel name, grid size, value in KiB) per dispatch of one rocprofv3
    counter CSV, in dispatch order."""
    import csv
    rows = []
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter:
                rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], int(r["Grid_Size"]),
                             float(r["Counter_Value"])))
    rows.sort()
    return [r[1:] for r in rows]


def summarize_pmc(args):
    """HBM bytes per attention launch from two counter passes.

    Each counter is scaled by the factor that makes it read the known size of
    the calibration copy (the largest copy-kernel dispatch of the run), so the
    result is in bytes whatever unit and coverage the counter has."""
    fetch = _counter_rows(args.summarize_pmc[0], "FETCH_SIZE")
    write = _counter_rows(args.summarize_pmc[1], "WRITE_SIZE")

    def calib(rows):
        copies = [r for r in rows if "copy" in r[0].lower()]
        if not copies:
            raise SystemExit("no copy-kernel dispatch in the counter CSV (run with --copy-calibration)")
        return max(c[2] for c in copies)

    meta = json.load(open(args.calibration_meta))
    first, count = meta["timed_dispatches"]

    def attn(rows):
        """Mean over the timed steps' attention dispatches."""
        names = [r[0] for r in rows if "attn_bf16_kernel" in r[0] or "attn_f32_kernel" in r[0]]
        if not names:
            raise SystemExit("no attention dispatch in the counter CSV")
        vals = [r[2] for r in rows if r[0] == names[0]][first:first + count]
        if len(vals) != count:
            raise SystemExit(f"expected {count} timed attention dispatches after {first}, "
                             f"found {len(vals)}")
        return float(np.mean(vals)), len(vals)

    known_kib = meta["copy_mib"] * 1024.0
    f_fetch = known_kib / calib(fetch)
    f_write = known_kib / calib(write)
    fk, nf = attn(fetch)
    wk, nw = attn(write)
    res = {
        "workload": meta["workload"],
        "kernel_source_sha": meta["kernel_source_sha"],
        "bytes_per_launch": round((fk * f_fetch + wk * f_write) * 1024.0),
        "fetch_bytes_per_launch": round(fk * f_fetch * 1024.0),
        "write_bytes_per_launch": round(wk * f_write * 1024.0),
        "algorithmic_bytes_per_launch": meta["algorithmic_bytes"],
        "raw_kib_per_launch": {"FETCH_SIZE": fk, "WRITE_SIZE": wk},
        "calibration": {"copy_mib": meta["copy_mib"], "fetch_factor": f_fetch, "write_factor": f_write},
        "dispatches": {"FETCH_SIZE": nf, "WRITE_SIZE": nw,
                       "which": f"the timed steps' attention launches: ordinals {first} to "
                                f"{first + count - 1} of the step's attention kernel"},
        "command": args.pmc_command,
    }
    with open(args.traffic_json or _traffic_path(meta["workload"]), "w") as f:
        json.dump(res, f, indent=1)
        f.write("\n")
    print(json.dumps(res))


def attention_roofline(flops, T, H, D, is_bf16, num_seqs):
    """(algorithmic bytes of one attention launch, whether HBM bounds it).

    Bytes: q, k, v read once, out written once, and cu_seqlens.  A bf16
    launch whose FLOPs per byte fall below the ridge point (peak bf16 FLOP/s
    over peak HBM bytes/s, 312.5) is HBM-bound; its roofline is then taken in
    GB/s.  The fp32 kernel is reported against the vector ALU."""
    elt = 2 if is_bf16 else 4
    nbytes = 4 * T * H * D * elt + 4 * (num_seqs + 1)
    ridge = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBPS * 1e9)
    return nbytes, bool(is_bf16 and flops / nbytes < ridge)


def cpu_baseline(wl, x, budget_s, causal=False):
    """Time the fp64 oracle (as it stands) on a bounded sample of the workload.

    The sample is whole segments (pre-pass + attention), taken in order until the
    time budget is spent; the throughput is scaled by the sample's own FLOPs."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    cu = x.cu_seqlens
    norm = (x.wq, x.wk) if wl.use_norm else (None, None)
    flops = 0.0
    nseg = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        i = nseg % wl.num_seqs
        a, b = int(cu[i]), int(cu[i + 1])
        q, k = oracle.qk_norm_rope(x.q[a:b], x.k[a:b], x.pos[a:b], wl.theta, *norm, wl.eps)
        oracle.segment_attention(q, k, x.v[a:b], wl.softmax_scale, causal)
        n = b - a
        flops += 4.0 * wl.H * wl.D * (n * (n + 1) / 2 if causal else n * n)
        nseg += 1
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{nseg} whole segments ({nseg / wl.num_seqs:.2f} passes over the batch), "
                      f"fp64 pre-pass + attention, {dt:.1f} s",
            "seconds": round(dt, 3), "blas": blas_backend()}


def blas_backend():
    """The BLAS library NumPy's matrix products run on, and its thread count."""
    try:
        from threadpoolctl import threadpool_info
        libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if libs:
            i = libs[0]
            return {"library": i.get("internal_api"), "version": i.get("version"),
                    "threads": i.get("num_threads"), "path": os.path.basename(i.get("filepath", ""))}
    except Exception:
        pass
    return None


def oracle_seconds_per_config(causal=False):
    """Wall-seconds of the whole fp64 oracle (pre-pass + attention) on each
    seeded workload: best of 3 for the two small ones, one run for the rest."""
    import oracle
    from vision_encoder_varlen_amd import workloads as W
    res = {}
    for n in (1, 2, 3, 4, 5):
        wl = W.config(n)
        x = W.generate(wl)
        norm = (x.wq, x.wk) if wl.use_norm else (None, None)
        best = None
        for _ in range(3 if n <= 2 else 1):
            t0 = time.perf_counter()
            q, k = oracle.qk_norm_rope(x.q, x.k, x.pos, wl.theta, *norm, wl.eps)
            oracle.varlen_attention(q, k, x.v, x.cu_seqlens, wl.softmax_scale, causal)
            dt = time.perf_counter() - t0
            best = dt if best is None else min(best, dt)
        res[wl.name] = {"seconds": round(best, 3),
                        "tflops": round(wl.attn_flops / best / 1e12, 4) if not causal else None}
        del x
    return res


def main():
    args = parse()
    if args.summarize_pmc:
        summarize_pmc(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (this path runs on a "
              "single GPU).", file=sys.stderr)
        sys.exit(2)
    # Step forms that exclude each other, refused before any GPU work.
    if args.fuse_q and args.fuse_qk:
        sys.exit("bench: --fuse-q and --fuse-qk are two forms of the step; pick one")
    if args.dense_batch and (args.fuse_q or args.fuse_qk):
        sys.exit("bench: --fuse-q / --fuse-qk time the work-list step; drop --dense-batch")

    import torch
    from vision_encoder_varlen_amd import _lib, ops
    from vision_encoder_varlen_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    lib = _lib.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    wl = W.config(args.config)
    x = W.generate(wl)
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    import ctypes
    # The step's inputs as a QKV projection leaves them (q_src, k_src, v), and
    # the attention's q and k, which the pre-pass writes from them every step:
    # the sources stay unchanged, so every step normalises and rotates the
    # same rows.
    if args.packed_qkv:
        # q_src, k_src, v as views of one packed [T, 3, H, D] projection output.
        qkv = torch.from_numpy(np.stack([x.q, x.k, x.v], axis=1)).to(tdt).to(dev)
        q_src, k_src, v = qkv[:, 0], qkv[:, 1], qkv[:, 2]
    else:
        q_src, k_src, v = (torch.from_numpy(a).to(tdt).to(dev) for a in (x.q, x.k, x.v))
    q = torch.empty(q_src.shape, dtype=tdt, device=dev)
    k = torch.empty(k_src.shape, dtype=tdt, device=dev)
    pos = torch.from_numpy(x.pos).to(dev)
    cu = torch.from_numpy(x.cu_seqlens).to(dev)
    wq = torch.from_numpy(x.wq).to(dev) if wl.use_norm else None
    wk = torch.from_numpy(x.wk).to(dev) if wl.use_norm else None
    wq_p = wq.data_ptr() if wq is not None else None
    wk_p = wk.data_ptr() if wk is not None else None
    out = torch.empty(q.shape, dtype=tdt, device=dev)
    T, H, D = q.shape
    # Token strides (elements): of q_src, k_src for the pre-pass, of q, k, v,
    # out for the attention; None = contiguous [T, H, D].
    src_strides = at_strides = None
    if args.packed_qkv:
        src_strides = (ctypes.c_int64 * 2)(q_src.stride(0), k_src.stride(0))
        at_strides = (ctypes.c_int64 * 4)(H * D, H * D, v.stride(0), H * D)
    dcode = ops.dtype_code(tdt)
    bm = ops.attn_block_m(H, D, tdt)
    plan = ops.varlen_worklist(cu, wl.max_seqlen, bm)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    check = _lib.check
    # Precomputed ctypes arguments keep host overhead per step far below GPU time.
    no_list = (None, 0, 0, 0, None, 0, None)
    wl_args = (cu.data_ptr(), wl.num_seqs, wl.max_seqlen, bm, plan.items.data_ptr(), plan.cap,
               plan.meta.data_ptr(), sh)
    # vit_qk_norm_rope_into: the pre-pass alone, and (the step's first
    # launch) the pre-pass with the work-list build; rope_mode 0: rotate-half.
    f_pre = f_fused = lib.vit_qk_norm_rope_into
    pre_head = (q_src.data_ptr(), k_src.data_ptr(), src_strides, q.data_ptr(), k.data_ptr(), T, H,
                D, dcode, pos.data_ptr(), float(wl.theta), wq_p, wk_p, float(wl.eps), 0, None)
    pre_args = pre_head + no_list + (sh,)
    fused_args = pre_head + wl_args
    f_wl, f_at = lib.vit_varlen_worklist, lib.vit_varlen_attn_planned
    flags = 1 if args.causal else 0     # VIT_ATTN_CAUSAL
    at_args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), cu.data_ptr(), plan.items.data_ptr(),
               plan.cap, plan.meta.data_ptr(), H, D, float(wl.softmax_scale), dcode, flags,
               out.data_ptr(), None, at_strides, sh)
    # The same attention call that also writes the log-sum-exp rows (timed
    # outside the timed loop, for its overhead).
    lse_buf = torch.empty((T, H), dtype=torch.float32, device=dev)
    at_lse_args = at_args[:-3] + (lse_buf.data_ptr(), at_strides, sh)
    if args.dense_batch:
        lens = np.diff(x.cu_seqlens)
        if len(set(lens.tolist())) != 1:
            sys.exit("bench: --dense-batch needs a workload of equal-length segments")
        f_at = lib.vit_dense_batch_attn
        at_args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), wl.num_seqs, int(lens[0]), H, D,
                   float(wl.softmax_scale), dcode, flags, out.data_ptr(), None, at_strides, sh)
        at_lse_args = at_args[:-3] + (lse_buf.data_ptr(), at_strides, sh)
    if args.fuse_q:
        if args.dense_batch:
            sys.exit("bench: --fuse-q times the work-list step; drop --dense-batch")
        # k's pre-pass with the work-list build in one launch; q's RMSNorm and
        # rotary inside the attention kernel, which reads q_src as it is.
        pre_head = (None, k_src.data_ptr(), src_strides, None, k.data_ptr(), T, H, D, dcode,
                    pos.data_ptr(), float(wl.theta), None, wk_p, float(wl.eps), 0, None)
        pre_args = pre_head + no_list + (sh,)
        fused_args = pre_head + wl_args
        f_at = lib.vit_varlen_attn_planned_qnorm_rope
        fq_strides = None
        if args.packed_qkv:
            fq_strides = (ctypes.c_int64 * 4)(q_src.stride(0), H * D, v.stride(0), H * D)
        at_args = (q_src.data_ptr(), k.data_ptr(), v.data_ptr(), cu.data_ptr(),
                   plan.items.data_ptr(), plan.cap, plan.meta.data_ptr(), H, D,
                   float(wl.softmax_scale), dcode, flags, pos.data_ptr(), float(wl.theta), wq_p,
                   float(wl.eps), 0, out.data_ptr(), None, fq_strides, sh)
        at_lse_args = at_args[:-3] + (lse_buf.data_ptr(), fq_strides, sh)
    if args.fuse_qk:
        if args.dense_batch or args.fuse_q:
            sys.exit("bench: --fuse-qk times the work-list step alone; drop --dense-batch / --fuse-q")
        # no pre-pass launch: the step's first launch builds the work-list, and
        # the attention kernel normalises and rotates q and k from q_src, k_src
        f_pre = f_fused = f_wl
        pre_args = fused_args = wl_args
        f_at = lib.vit_varlen_attn_planned_qk_norm_rope
        fqk_strides = None
        if args.packed_qkv:
            fqk_strides = (ctypes.c_int64 * 4)(q_src.stride(0), k_src.stride(0), v.stride(0), H * D)
        at_args = (q_src.data_ptr(), k_src.data_ptr(), v.data_ptr(), cu.data_ptr(),
                   plan.items.data_ptr(), plan.cap, plan.meta.data_ptr(), H, D,
                   float(wl.softmax_scale), dcode, flags, pos.data_ptr(), float(wl.theta), wq_p,
                   wk_p, float(wl.eps), 0, out.data_ptr(), None, fqk_strides, sh)
        at_lse_args = at_args[:-3] + (lse_buf.data_ptr(), fqk_strides, sh)

    if args.copy_calibration > 0:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    K, Wm = args.steps, args.warmup
    f_hook = lib.vit_time_next_kernel

    def new_events(n):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        for e in evs:          # torch creates the HIP event on its first record
            e.record(stream)
        return evs

    # e[0] / e[1]: the attention kernel's own dispatch start and end, taken on
    # every hook_every-th step of the timed loop (a hooked launch records two
    # more events, which adds a gap before the next launch).
    every = max(1, args.hook_every)
    ev = [new_events(2) if i % every == 0 else None for i in range(K)]
    torch.cuda.synchronize()

    def step(e=None):
        if args.dense_batch:      # no work-list to build
            check(f_pre(*pre_args))
        else:
            check(f_fused(*fused_args))
        if e is not None:
            check(f_hook(e[0].cuda_event, e[1].cuda_event))
        check(f_at(*at_args))

    settle_steps, settle_ms = settle(step, args.settle_ms, torch)
    for _ in range(Wm):
        step()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(K):
        step(ev[i])
    end.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    if args.copy_calibration > 0 and args.calibration_meta:
        # the timed steps' attention launches, as ordinals among the dispatches
        # of the step's attention kernel (the first attention kernel the run
        # dispatches): the settle and warm-up steps come before them, the
        # side loops after
        with open(args.calibration_meta, "w") as f:
            json.dump({"copy_mib": args.copy_calibration, "workload": wl.name,
                       "kernel_source_sha": _kernel_sha(),
                       "algorithmic_bytes": 4 * T * H * D * q.element_size(),
                       "timed_dispatches": [settle_steps + Wm, K]}, f)
    ms_per_step = total_ms / K
    attn_avg_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev if e is not None]))

    # Outside the timed region: each other kernel's own duration, from the
    # same dispatch-timestamp events, one kernel per loop (a kernel queued
    # behind a different, still-running one would count part of its wait).
    attn_samples = [e[0].elapsed_time(e[1]) for e in ev if e is not None]
    attn_med_ms = float(np.median(attn_samples))

    # A buffer read before each memory-bound launch, so the launch reads its
    # inputs from HBM rather than from the Infinity Cache (256 MB) that the
    # previous launch of the same small inputs left them in.  Reading (not
    # writing) leaves the caches holding clean lines, so the timed launch does
    # not also pay for writing a previous kernel's dirty lines back.
    flush = torch.ones(max(1, args.flush_mib) << 18, dtype=torch.float32, device=dev)

    def side_loop(fn, fargs, flushed=False):
        """(mean, median) ms of one kernel's own dispatch, K launches."""
        evs = [new_events(2) for _ in range(K)]
        torch.cuda.synchronize()
        for i, e in enumerate(evs):
            if flushed:
                flush.sum()
            check(f_hook(e[0].cuda_event, e[1].cuda_event))
            check(fn(*fargs))
        torch.cuda.synchronize()
        t = [e[0].elapsed_time(e[1]) for e in evs]
        return float(np.mean(t)), float(np.median(t))

    pre_avg_ms, pre_med_ms = side_loop(f_pre, pre_args, flushed=True)
    pre_warm_ms, _ = side_loop(f_pre, pre_args)
    wl_avg_ms, _ = side_loop(f_wl, wl_args)
    fused_avg_ms, _ = side_loop(f_fused, fused_args)
    lse_avg_ms, _ = side_loop(f_at, at_lse_args)
    attn_cold_ms, attn_cold_med_ms = side_loop(f_at, at_args, flushed=True)
    del flush

    ceiling = mfma_ceiling(lib, torch, dev, stream) if is_bf16_dtype(wl) else None

    # Correctness guard on the measured buffers: finite output, no work-list errors.
    meta = plan.meta.cpu().numpy()
    if int(meta[1]) != 0 or not torch.isfinite(out).all().item():
        print("bench: work-list error or non-finite output", file=sys.stderr)
        sys.exit(3)

    flops = wl.attn_flops
    if args.causal:
        s_len = np.diff(x.cu_seqlens).astype(np.float64)
        flops = 4.0 * H * D * float(np.sum(s_len * (s_len + 1) / 2))
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (attn_avg_ms * 1e-3) / 1e12
    is_bf16 = wl.dtype == "bf16"
    peak = PEAK_BF16_TFLOPS if is_bf16 else PEAK_F32_VALU_TFLOPS
    traffic = None
    tpath = args.traffic_json or _traffic_path(wl.name)
    if os.path.exists(tpath):
        try:
            tj = json.load(open(tpath))
            if tj.get("workload") == wl.name and tj.get("kernel_source_sha") == _kernel_sha():
                traffic = tj.get("bytes_per_launch")
        except Exception:
            traffic = None
    attn_bytes, hbm_bound = attention_roofline(flops, T, H, D, is_bf16, wl.num_seqs)
    tensors = 1 if args.fuse_q else 2     # q and k, or k alone
    pre_bytes = 2 * tensors * T * H * D * (2 if is_bf16 else 4) + 8 * T + \
        (4 * tensors * D if wl.use_norm else 0)
    pre_gbps = pre_bytes / (pre_avg_ms * 1e-3) / 1e9
    pre_med_gbps = pre_bytes / (pre_med_ms * 1e-3) / 1e9

    result = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "settle": {"steps": settle_steps, "ms": round(settle_ms, 1),
                   "note": "untimed steps before the warm-up steps, until the clock has ramped"},
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if is_bf16 else "f32",
        "data": "synthetic",
        "config": {"workload": wl.name + ("_packed_qkv" if args.packed_qkv else "")
                   + ("_dense_batch" if args.dense_batch else "")
                   + ("_causal" if args.causal else "")
                   + ("_fused_q" if args.fuse_q else "")
                   + ("_fused_qk" if args.fuse_qk else ""),
                   "images": wl.num_seqs, "tokens": T, "heads": H,
                   "head_dim": D, "max_seqlen": wl.max_seqlen, "qk_norm": wl.use_norm,
                   "rope": "2d", "flops_per_step": flops, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma" if is_bf16 else "alu", "kernel": "attn_bf16" if is_bf16 else "attn_f32",
                     "achieved": round(achieved, 3), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4), "traffic": traffic,
                     "avg_launch_us": round(attn_avg_ms * 1e3, 3),
                     "median_launch_us": round(attn_med_ms * 1e3, 3),
                     "timed_samples": len(attn_samples),
                     "algorithmic_bytes": attn_bytes,
                     "flop_per_byte": round(flops / attn_bytes, 2)},
        "kernels_us": {"prepass_and_worklist_launch": round(fused_avg_ms * 1e3, 3),
                       "prepass_alone": round(pre_avg_ms * 1e3, 3),
                       "worklist_alone": round(wl_avg_ms * 1e3, 3),
                       "attention": round(attn_avg_ms * 1e3, 3),
                       "attention_median": round(attn_med_ms * 1e3, 3),
                       "attention_after_cache_flush": round(attn_cold_ms * 1e3, 3),
                       "attention_after_cache_flush_median": round(attn_cold_med_ms * 1e3, 3),
                       "attention_with_lse": round(lse_avg_ms * 1e3, 3),
                       "prepass_cache_warm": round(pre_warm_ms * 1e3, 3)},
        "prepass": {"bound": "hbm", "achieved": round(pre_gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                    "frac": round(pre_gbps / PEAK_HBM_GBPS, 4), "bytes_per_launch": pre_bytes,
                    "avg_launch_us": round(pre_avg_ms * 1e3, 3),
                    "median_launch_us": round(pre_med_ms * 1e3, 3),
                    "median_achieved": round(pre_med_gbps, 1),
                    "timing": f"each launch after a {args.flush_mib} MiB buffer read (inputs from HBM)"},
        "step_frac_of_peak": round(value / peak, 4),
    }
    if hbm_bound:
        gbps = attn_bytes / (attn_avg_ms * 1e-3) / 1e9
        result["roofline"].update({"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS,
                                   "unit": "GB/s", "frac": round(gbps / PEAK_HBM_GBPS, 4),
                                   "achieved_tflops": round(achieved, 3),
                                   "frac_of_bf16_peak": round(achieved / peak, 4)})
    if is_bf16:
        result["peak_on_box"] = peak_on_box(torch, dev)
    if ceiling is not None:
        result["mfma_ceiling"] = ceiling
        if not hbm_bound:
            result["roofline"]["frac_of_random_operand_ceiling"] = round(achieved / ceiling["random_bf16"], 4)
    if args.fuse_qk:
        # no pre-pass kernel to report: the side loops above timed the work-list build
        result["prepass"] = {"note": "none: q and k are normalised and rotated inside the "
                                     "attention kernel (vit_varlen_attn_planned_qk_norm_rope)"}
        result["kernels_us"] = {k: v for k, v in result["kernels_us"].items()
                                if k not in ("prepass_alone", "prepass_cache_warm",
                                             "prepass_and_worklist_launch")}
    if args.second_target and args.config == 2 and not (args.causal or args.fuse_q or args.dense_batch
                                                         or args.packed_qkv or args.fuse_qk):
        result["second_target"] = second_target(args.second_target, lib, torch, dev, stream,
                                                max(K, 50), new_events, args.settle_ms)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, x, args.cpu_seconds, args.causal)
        if not args.no_oracle_per_config:
            result["cpu_baseline"]["oracle_seconds_per_config"] = oracle_seconds_per_config(args.causal)
    print(json.dumps(result), flush=True)


def settle(step, ms, torch):
    """Run `step` untimed, in groups of 10 with a synchronisation after each,
    until at least `ms` milliseconds of wall time have passed; returns the
    number of steps and the milliseconds taken.  Under sustained load the
    chip's clock climbs for a few hundred milliseconds: MFMA-bound launches
    of the 1 x 16384 workload run about 1.53 ms at first and 1.21 ms once it
    has settled."""
    n, t0 = 0, time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(10):
            step()
        n += 10
        torch.cuda.synchronize()
    return n, (time.perf_counter() - t0) * 1e3


def second_target(n, lib, torch, dev, stream, launches, new_events, settle_ms):
    """The attention kernel alone on seeded workload n, as the step runs it
    (pre-pass applied once, then the planned attention): its own dispatch
    duration over `launches` launches, and the fraction of bf16 MFMA peak."""
    from vision_encoder_varlen_amd import _lib, ops
    from vision_encoder_varlen_amd import workloads as W
    wl = W.config(n)
    x = W.generate(wl)
    q, k, v = (torch.from_numpy(a).to(torch.bfloat16).to(dev) for a in (x.q, x.k, x.v))
    pos = torch.from_numpy(x.pos).to(dev)
    cu = torch.from_numpy(x.cu_seqlens).to(dev)
    wq = torch.from_numpy(x.wq).to(dev) if wl.use_norm else None
    wk = torch.from_numpy(x.wk).to(dev) if wl.use_norm else None
    T, H, D = q.shape
    ops.qk_norm_rope_(q, k, pos, wl.theta, wq, wk, wl.eps)
    plan = ops.varlen_worklist(cu, wl.max_seqlen, ops.attn_block_m(H, D, q.dtype))
    out = torch.empty_like(q)
    sh = stream.cuda_stream
    at_args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), cu.data_ptr(), plan.items.data_ptr(),
               plan.cap, plan.meta.data_ptr(), H, D, float(wl.softmax_scale), _lib.VIT_BF16, 0,
               out.data_ptr(), None, None, sh)
    settled, settled_ms = settle(lambda: _lib.check(lib.vit_varlen_attn_planned(*at_args)),
                                 settle_ms, torch)
    evs = [new_events(2) for _ in range(launches)]
    torch.cuda.synchronize()
    for e in evs:
        _lib.check(lib.vit_time_next_kernel(e[0].cuda_event, e[1].cuda_event))
        _lib.check(lib.vit_varlen_attn_planned(*at_args))
    torch.cuda.synchronize()
    if int(plan.meta.cpu()[1]) != 0 or not torch.isfinite(out).all().item():
        print("bench: second target: work-list error or non-finite output", file=sys.stderr)
        sys.exit(3)
    t = [e[0].elapsed_time(e[1]) for e in evs]
    avg, med = float(np.mean(t)), float(np.median(t))
    ach = wl.attn_flops / (avg * 1e-3) / 1e12
    return {"workload": wl.name, "tokens": T, "heads": H, "head_dim": D, "images": wl.num_seqs,
            "flops_per_launch": wl.attn_flops, "launches": launches,
            "settle": {"launches": settled, "ms": round(settled_ms, 1)},
            "attention_avg_us": round(avg * 1e3, 3), "attention_median_us": round(med * 1e3, 3),
            "achieved": round(ach, 3), "unit": "TFLOP/s", "peak": PEAK_BF16_TFLOPS,
            "frac": round(ach / PEAK_BF16_TFLOPS, 4),
            "median_frac": round(wl.attn_flops / (med * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}


def is_bf16_dtype(wl):
    return wl.dtype == "bf16"


def mfma_ceiling(lib, torch, dev, stream):
    """Sustained bf16 MFMA rate of a kernel that does nothing but MFMAs, on
    operands drawn like the workload's inputs (N(0,1) rounded to bf16) and on
    zeros.  The chip lowers its clock when operands toggle many bits, so the
    first figure is what any bf16 MFMA kernel can reach on such data."""
    from vision_encoder_varlen_amd import _lib
    probe = _lib.load_probe()   # libvit_probe.so: measurement support, not the path
    nbytes = 4 << 20
    gen = torch.Generator(device="cpu").manual_seed(0)
    rnd = torch.randn(nbytes // 2, generator=gen).to(torch.bfloat16).to(dev)
    zero = torch.zeros(nbytes // 2, dtype=torch.bfloat16, device=dev)
    blocks, iters = 512, 1500
    sink = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    flops = blocks * 4 * 32 * iters * 32768.0
    out = {}
    for name, buf in (("random_bf16", rnd), ("zeros", zero)):
        times = []
        for _ in range(5):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            rc = probe.vit_probe_mfma(buf.data_ptr(), nbytes, blocks, iters, sink.data_ptr(),
                                      stream.cuda_stream)
            if rc != 0:
                raise RuntimeError(f"vit_probe_mfma: {probe.vit_probe_last_error().decode()}")
            e1.record(stream)
            e1.synchronize()
            times.append(e0.elapsed_time(e1))
        best = min(times[2:])  # the clock settles over the first launches
        out[name] = round(flops / (best * 1e-3) / 1e12, 1)
    out["unit"] = "TFLOP/s"
    out["probe"] = ("vit_probe_mfma (libvit_probe.so): 512 workgroups x 4 waves, 4 independent "
                    "32x32x16 bf16 chains per wave")
    return out


def peak_on_box(torch, dev):
    """Dense bf16 MFMA peak computed on this machine: CUs x peak shader clock x
    4096 FLOP per CU per clock.  Reads the clock and CU count through the HIP
    runtime the process already has loaded (hipDeviceGetAttribute with
    hipDeviceAttributeClockRate = 5, kHz, and
    hipDeviceAttributeMultiprocessorCount = 63, the values of ROCm's
    hip_runtime_api.h); None if the CU count read that way disagrees with
    torch's (a sign of other enum values)."""
    import ctypes
    paths = sorted({line.split()[-1] for line in open("/proc/self/maps") if "libamdhip64" in line})
    if not paths:
        return None
    hip = ctypes.CDLL(paths[0])
    get = hip.hipDeviceGetAttribute
    get.argtypes = [ctypes.POINTER(ctypes.c_int), ctypes.c_int, ctypes.c_int]
    get.restype = ctypes.c_int
    idx = dev.index if dev.index is not None else 0
    clk, cus = ctypes.c_int(0), ctypes.c_int(0)
    if get(ctypes.byref(clk), 5, idx) != 0 or get(ctypes.byref(cus), 63, idx) != 0:
        return None
    if cus.value != torch.cuda.get_device_properties(idx).multi_processor_count:
        return None
    return {"cus": cus.value, "max_clock_mhz": round(clk.value / 1e3, 1),
            "bf16_dense_tflops": round(cus.value * clk.value * 1e3 * 4096 / 1e12, 1),
            "formula": "CUs x peak shader clock x 4096 bf16 FLOP per CU per clock"}


def _traffic_path(workload):
    return os.path.join(ROOT, "profiles", f"attn_traffic_{workload}.json")


def _kernel_sha():
    """Hash of the attention kernel's sources (the kernel and its launch header)."""
    import hashlib
    h = hashlib.sha256()
    for name in ("attn_bf16.hip", "attn_bf16_kernel.h", "vit_kernels.h"):
        with open(os.path.join(ROOT, "vision_encoder_varlen_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


if __name__ == "__main__":
    main()
