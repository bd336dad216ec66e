"""Pins for the CPU work-list rule (hand-derived cases and brute-force properties)."""
import itertools
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worklist_cases.json")


def test_hand_derived_cases():
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    assert len(cases) >= 5
    for c in cases:
        items, count, err = oracle.worklist(np.asarray(c["cu_seqlens"], dtype=np.int64), c["block_m"],
                                            c.get("max_seqlen"))
        assert count == len(c["items"]), c["name"]
        assert items.tolist() == c["items"], c["name"]
        assert err == c["err"], c["name"]


@pytest.mark.parametrize("seed", range(20))
def test_brute_force_properties(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(0, 40))
    lens = rng.integers(0, 700, size=n)
    lens[rng.random(n) < 0.2] = 0
    if n > 3:
        lens[1] = lens[2]               # force a tie
    cu = np.concatenate([[0], np.cumsum(lens)])
    bm = int(rng.choice([32, 64, 128]))
    items, count, err = oracle.worklist(cu, bm, int(lens.max()) if n else 0)
    assert err == 0
    # every (segment, tile) exactly once
    want = {(i, j) for i in range(n) for j in range(-(-int(lens[i]) // bm))}
    got = [tuple(x) for x in items.tolist()]
    assert len(got) == len(set(got)) == len(want) == count
    assert set(got) == want
    # longest first, ties by segment index, tiles ascending inside a segment
    key = [(-int(lens[i]), i, j) for i, j in got]
    assert key == sorted(key)
    # each segment's tiles are contiguous in the list
    for _, grp in itertools.groupby(got, key=lambda x: x[0]):
        js = [j for _, j in grp]
        assert js == list(range(len(js)))


def test_validation_errors():
    _, count, err = oracle.worklist([3, 5, 9], 64, 100)
    assert count == 0 and err == 1
    items, count, err = oracle.worklist([0, 5, 3, 9], 64, 100)
    assert err == 2 and items.tolist() == [[2, 0], [0, 0]]
    items, count, err = oracle.worklist([0, 5, 300, 310], 128, 100)
    assert err == 4 and items.tolist() == [[2, 0], [0, 0]]
    items, count, err = oracle.worklist([0], 64, 0)
    assert count == 0 and err == 0
