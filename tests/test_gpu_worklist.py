"""Device work-list builder vs the CPU rule: bit-exact items, count and error bits."""
import json
import os

import numpy as np
import pytest

import oracle
from vision_encoder_varlen_amd import workloads as W

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worklist_cases.json")


def _device_list(cu, block_m, max_seqlen, cap=None):
    import torch
    from vision_encoder_varlen_amd import ops
    cu_t = torch.from_numpy(np.asarray(cu, dtype=np.int32)).cuda()
    plan = ops.varlen_worklist(cu_t, max_seqlen, block_m, cap=cap)
    meta = plan.meta.cpu().numpy()
    count = int(meta[0])
    items = plan.items.cpu().numpy()[:count]
    return items, count, int(meta[1])


def _check(cu, block_m, max_seqlen):
    want_items, want_count, want_err = oracle.worklist(np.asarray(cu), block_m, max_seqlen)
    items, count, err = _device_list(cu, block_m, max_seqlen)
    assert count == want_count
    assert err == want_err
    assert np.array_equal(items, want_items)


def test_hand_derived_cases():
    cases = json.load(open(GOLDEN))["cases"]
    for c in cases:
        if len(c["cu_seqlens"]) < 1:
            continue
        _check(c["cu_seqlens"], c["block_m"], c["max_seqlen"])


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
def test_workload_lists(n):
    wl = W.config(n)
    for bm in (32, 128):
        _check(wl.cu_seqlens, bm, wl.max_seqlen)


@pytest.mark.parametrize("seed", range(6))
def test_random_ragged_with_ties_and_empties(seed):
    rng = np.random.default_rng(1000 + seed)
    n = int(rng.choice([7, 63, 64, 65, 1000, 4097]))
    lens = rng.integers(0, 300, size=n)
    lens[rng.random(n) < 0.1] = 0
    lens[rng.random(n) < 0.3] = 128            # many ties
    cu = np.concatenate([[0], np.cumsum(lens)])
    _check(cu, 128, int(lens.max()))
    _check(cu, 32, int(lens.max()))


def test_maximum_segment_count():
    rng = np.random.default_rng(5)
    lens = rng.integers(1, 50, size=8192)
    cu = np.concatenate([[0], np.cumsum(lens)])
    _check(cu, 128, 49)


def test_understated_max_seqlen_flags_and_skips():
    cu = [0, 10, 500, 505]
    items, count, err = _device_list(cu, 64, 100)
    assert err == 4 and items.tolist() == [[0, 0], [2, 0]]


def test_negative_length_and_bad_origin():
    _check([0, 10, 4, 20], 64, 100)
    _check([1, 5], 64, 4)
