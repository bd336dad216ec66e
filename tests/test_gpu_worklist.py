"""Device work-list builder vs the CPU rule: bit-exact items, count and error bits.

Each device item is four int32, (segment, q-tile, first token, length): the
first two are the list the CPU rule gives; the last two are read off the
input cu_seqlens; the rows after the count, up to 2048 of them (or the
capacity), must carry segment -1.
"""
import json
import os

import numpy as np
import pytest

import oracle
from vision_encoder_varlen_amd import workloads as W

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worklist_cases.json")


SENTINEL_SPAN = 2048


def _device_list(cu, block_m, max_seqlen, cap=None):
    """(segment, q-tile) rows, count and error bits of a device list, after
    checking its other two columns and the marked rows after the count."""
    import torch
    from vision_encoder_varlen_amd import ops
    cu = np.asarray(cu, dtype=np.int64)
    cu_t = torch.from_numpy(cu.astype(np.int32)).cuda()
    plan = ops.varlen_worklist(cu_t, max_seqlen, block_m, cap=cap)
    meta = plan.meta.cpu().numpy()
    count = int(meta[0])
    full = plan.items.cpu().numpy()
    items = full[:count]
    seg = items[:, 0].astype(np.int64)
    assert np.array_equal(items[:, 2], cu[seg]), "first-token column"
    assert np.array_equal(items[:, 3], cu[seg + 1] - cu[seg]), "length column"
    marked = full[count:min(plan.cap, count + SENTINEL_SPAN)]
    assert np.all(marked[:, 0] == -1), "rows after the count must carry segment -1"
    return items[:, :2], count, int(meta[1])


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
