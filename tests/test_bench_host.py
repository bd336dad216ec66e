"""bench.py's host-side parts, without a GPU: the one-GPU rule, the roofline
each workload is judged against, and the HBM-traffic summary of two
rocprofv3 counter passes."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from vision_encoder_varlen_amd import workloads as W  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr or "single GPU" in r.stderr
    assert r.stdout == ""


@pytest.mark.parametrize("flags", [["--fuse-q", "--fuse-qk"], ["--fuse-qk", "--dense-batch"],
                                   ["--fuse-q", "--dense-batch"]])
def test_exclusive_step_forms_are_refused_before_any_gpu_work(flags):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *flags],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "bench:" in r.stderr
    assert r.stdout == ""


@pytest.mark.parametrize("cfg,bound", [(2, "mfma"), (3, "mfma"), (4, "mfma"), (5, "hbm")])
def test_roofline_bound_per_workload(cfg, bound):
    wl = W.config(cfg)
    T, H, D = wl.total_tokens, wl.H, wl.D
    nbytes, hbm = bench.attention_roofline(wl.attn_flops, T, H, D, True, wl.num_seqs)
    # q, k, v and out once in bf16, plus cu_seqlens
    assert nbytes == 4 * T * H * D * 2 + 4 * (wl.num_seqs + 1)
    assert ("hbm" if hbm else "mfma") == bound
    # the bf16 ridge point: 2.5e15 FLOP/s over 8e12 B/s
    assert (wl.attn_flops / nbytes < 312.5) == hbm


def test_fp32_kernel_is_never_reported_as_hbm_bound():
    wl = W.config(1)
    _, hbm = bench.attention_roofline(wl.attn_flops, wl.total_tokens, wl.H, wl.D, False,
                                      wl.num_seqs)
    assert not hbm


def _counter_csv(path, counter, rows):
    """rows: (kernel name, value), in dispatch order; written to the file in
    reverse, so that the reader has to sort them by dispatch id."""
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Grid_Size",
                                          "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (name, value) in reversed(list(enumerate(rows))):
            w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": name, "Grid_Size": 256,
                        "Counter_Name": counter, "Counter_Value": value})


def test_pmc_summary_scales_each_counter_by_the_calibration_copy(tmp_path):
    # The copy of 64 MiB reads FETCH_SIZE = 32768 KiB (factor 2) and
    # WRITE_SIZE = 65536 KiB (factor 1); the two timed attention dispatches
    # (ordinals 1 and 2 of the step's attention kernel) average 1000 KiB
    # fetched and 300 KiB written.  The warm-up dispatch before them, the
    # side-loop dispatch after them and another attention kernel's dispatch
    # are left out.
    fetch, write = tmp_path / "fetch.csv", tmp_path / "write.csv"
    attn = "void vit::attn_bf16_kernel<Cfg<80>>(...)"
    other = "void vit::attn_bf16_kernel<Cfg<128>>(...)"
    _counter_csv(fetch, "FETCH_SIZE", [("__amd_rocclr_copyBuffer", 32768.0), ("prepass_kernel", 5.0),
                                       (attn, 7000.0), ("prepass_kernel", 5.0), (attn, 900.0),
                                       ("prepass_kernel", 5.0), (attn, 1100.0), (attn, 9000.0),
                                       (other, 8000.0)])
    _counter_csv(write, "WRITE_SIZE", [("__amd_rocclr_copyBuffer", 65536.0), (attn, 700.0),
                                       (attn, 300.0), (attn, 300.0), (attn, 900.0)])
    meta = tmp_path / "meta.json"
    meta.write_text(json.dumps({"copy_mib": 64, "workload": "w", "kernel_source_sha": "x",
                                "algorithmic_bytes": 123, "timed_dispatches": [1, 2]}))
    out = tmp_path / "traffic.json"
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--summarize-pmc",
                        str(fetch), str(write), "--calibration-meta", str(meta),
                        "--traffic-json", str(out)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    res = json.loads(out.read_text())
    assert res["fetch_bytes_per_launch"] == 1000 * 2 * 1024
    assert res["write_bytes_per_launch"] == 300 * 1 * 1024
    assert res["bytes_per_launch"] == (2000 + 300) * 1024
    assert res["dispatches"]["FETCH_SIZE"] == 2 and res["dispatches"]["WRITE_SIZE"] == 2
    assert res["algorithmic_bytes_per_launch"] == 123
