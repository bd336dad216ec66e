"""Pins for the oracle's attention against things other than itself.

* the dense block-diagonal-mask formulation of ``VisionAttention.forward`` on the
  vLLM page ``vllm.models.dots3_note.nvidia.vision_attention`` (a different
  computation: one softmax over all T keys with off-block entries excluded);
* PyTorch's ``scaled_dot_product_attention`` in float64 on the CPU with a
  boolean block-diagonal mask (a library routine);
* pure-Python brute force with ``math.exp`` on tiny inputs;
* closed forms and invariants (length-1 segment, constant V, zero scale, key
  shift, hard-attention limit, permutations, segment isolation).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as oattn


def _rand(rng, T, H, D):
    return rng.standard_normal((T, H, D))


def _cu(lens):
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)


def _dense_mask_attention(q, k, v, cu, scale):
    """``VisionAttention.forward``: full T x T scores, excluded outside diagonal blocks."""
    T, H, D = q.shape
    allowed = np.zeros((T, T), dtype=bool)
    for i in range(len(cu) - 1):
        allowed[cu[i]:cu[i + 1], cu[i]:cu[i + 1]] = True
    out = np.full((T, H, D), np.nan)
    for h in range(H):
        s = (q[:, h, :] @ k[:, h, :].T) * scale
        s = np.where(allowed, s, -np.inf)
        rows = allowed.any(axis=1)
        s = s[rows]
        e = np.exp(s - s.max(axis=1, keepdims=True))
        p = e / e.sum(axis=1, keepdims=True)
        out[rows, h, :] = p @ v[:, h, :]
    return out


LAYOUTS = [[5], [1, 7, 3], [4, 0, 9, 1], [16, 48, 1], [2, 2, 2, 2, 2], [31, 1, 0, 13]]


@pytest.mark.parametrize("lens", LAYOUTS)
def test_matches_dense_block_mask(lens):
    rng = np.random.default_rng(sum(lens) + len(lens))
    cu = _cu(lens)
    T = int(cu[-1])
    q, k, v = (_rand(rng, T, 2, 8) for _ in range(3))
    got = oracle.varlen_attention(q, k, v, cu, 0.37)
    want = _dense_mask_attention(q, k, v, cu, 0.37)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("lens", LAYOUTS)
def test_matches_torch_sdpa_float64(lens):
    rng = np.random.default_rng(100 + sum(lens))
    cu = _cu(lens)
    T = int(cu[-1])
    H, D = 3, 16
    q, k, v = (_rand(rng, T, H, D) for _ in range(3))
    scale = 1.0 / math.sqrt(D)
    mask = torch.zeros((T, T), dtype=torch.bool)
    for i in range(len(cu) - 1):
        mask[cu[i]:cu[i + 1], cu[i]:cu[i + 1]] = True
    tq, tk, tv = (torch.from_numpy(x).permute(1, 0, 2).contiguous() for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=mask, scale=scale).permute(1, 0, 2).numpy()
    got = oracle.varlen_attention(q, k, v, cu, scale)
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-12)


def test_brute_force_python_loops():
    rng = np.random.default_rng(7)
    lens = [3, 1, 4]
    cu = _cu(lens)
    T, H, D = int(cu[-1]), 2, 4
    q, k, v = (_rand(rng, T, H, D) for _ in range(3))
    scale = 0.8
    want = np.zeros((T, H, D))
    for i in range(len(lens)):
        a, b = cu[i], cu[i + 1]
        for h in range(H):
            for t in range(a, b):
                logits = [scale * sum(q[t, h, d] * k[u, h, d] for d in range(D)) for u in range(a, b)]
                mx = max(logits)
                w = [math.exp(x - mx) for x in logits]
                z = sum(w)
                for d in range(D):
                    want[t, h, d] = sum(w[j] * v[a + j, h, d] for j in range(b - a)) / z
    got = oracle.varlen_attention(q, k, v, cu, scale)
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-14)


def test_length_one_segment_returns_its_value_row_exactly():
    rng = np.random.default_rng(1)
    cu = _cu([5, 1, 6])
    q, k, v = (_rand(rng, 12, 2, 8) for _ in range(3))
    out = oracle.varlen_attention(q, k, v, cu, 0.5)
    assert np.array_equal(out[5], v[5])


def test_constant_values_give_the_constant():
    rng = np.random.default_rng(2)
    cu = _cu([9, 20])
    q, k = _rand(rng, 29, 2, 8), _rand(rng, 29, 2, 8)
    v = np.empty((29, 2, 8))
    v[:9] = rng.standard_normal((1, 2, 8))
    v[9:] = rng.standard_normal((1, 2, 8))
    out = oracle.varlen_attention(q, k, v, cu, 1.3)
    np.testing.assert_allclose(out, v, rtol=0, atol=1e-14)


def test_zero_scale_is_the_segment_mean():
    rng = np.random.default_rng(3)
    cu = _cu([7, 13])
    q, k, v = (_rand(rng, 20, 2, 8) for _ in range(3))
    out = oracle.varlen_attention(q, k, v, cu, 0.0)
    np.testing.assert_allclose(out[:7], np.broadcast_to(v[:7].mean(0), (7, 2, 8)), atol=1e-14)
    np.testing.assert_allclose(out[7:], np.broadcast_to(v[7:].mean(0), (13, 2, 8)), atol=1e-14)


def test_key_shift_invariance():
    """Adding one vector to every key of a segment adds a per-row constant to the logits."""
    rng = np.random.default_rng(4)
    cu = _cu([11, 6])
    q, k, v = (_rand(rng, 17, 2, 8) for _ in range(3))
    k2 = k.copy()
    k2[:11] += rng.standard_normal((1, 2, 8))
    a = oracle.varlen_attention(q, k, v, cu, 0.4)
    b = oracle.varlen_attention(q, k2, v, cu, 0.4)
    np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-12)


def test_hard_attention_limit_picks_the_argmax_key():
    rng = np.random.default_rng(5)
    cu = _cu([10])
    q, k, v = (_rand(rng, 10, 1, 8) for _ in range(3))
    out = oracle.varlen_attention(q, k, v, cu, 1e6)
    best = np.argmax(q[:, 0, :] @ k[:, 0, :].T, axis=1)
    np.testing.assert_allclose(out[:, 0, :], v[best, 0, :], atol=1e-12)


def test_output_is_a_convex_combination_of_values():
    rng = np.random.default_rng(6)
    cu = _cu([8, 25])
    q, k, v = (_rand(rng, 33, 2, 4) for _ in range(3))
    out = oracle.varlen_attention(q, k, v, cu, 2.0)
    for a, b in ((0, 8), (8, 33)):
        assert np.all(out[a:b] <= v[a:b].max(0) + 1e-12)
        assert np.all(out[a:b] >= v[a:b].min(0) - 1e-12)


def test_segment_permutation_permutes_outputs():
    rng = np.random.default_rng(8)
    lens = [3, 8, 5]
    cu = _cu(lens)
    q, k, v = (_rand(rng, 16, 2, 8) for _ in range(3))
    out = oracle.varlen_attention(q, k, v, cu, 0.3)
    order = [2, 0, 1]
    idx = np.concatenate([np.arange(cu[i], cu[i + 1]) for i in order])
    cu2 = _cu([lens[i] for i in order])
    out2 = oracle.varlen_attention(q[idx], k[idx], v[idx], cu2, 0.3)
    np.testing.assert_allclose(out2, out[idx], rtol=1e-13, atol=1e-14)


def test_head_permutation_permutes_outputs():
    rng = np.random.default_rng(9)
    cu = _cu([6, 9])
    q, k, v = (_rand(rng, 15, 4, 8) for _ in range(3))
    perm = [3, 1, 0, 2]
    a = oracle.varlen_attention(q, k, v, cu, 0.3)
    b = oracle.varlen_attention(q[:, perm], k[:, perm], v[:, perm], cu, 0.3)
    np.testing.assert_allclose(b, a[:, perm], rtol=1e-13, atol=1e-14)


def test_segment_isolation_is_bit_exact():
    rng = np.random.default_rng(10)
    cu = _cu([6, 9, 4])
    q, k, v = (_rand(rng, 19, 2, 8) for _ in range(3))
    a = oracle.varlen_attention(q, k, v, cu, 0.3)
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    for x in (q2, k2, v2):
        x[6:15] += 1.0
    b = oracle.varlen_attention(q2, k2, v2, cu, 0.3)
    assert np.array_equal(a[:6], b[:6]) and np.array_equal(a[15:], b[15:])
    assert not np.allclose(a[6:15], b[6:15])


def test_row_sampler_matches_full_and_blocks_do_not_change_rows(monkeypatch):
    rng = np.random.default_rng(11)
    cu = _cu([40, 3, 77])
    q, k, v = (_rand(rng, 120, 2, 8) for _ in range(3))
    full = oracle.varlen_attention(q, k, v, cu, 0.25)
    tok = rng.integers(0, 120, size=30)
    hd = rng.integers(0, 2, size=30)
    rows = oracle.varlen_attention_rows(q, k, v, cu, 0.25, tok, hd)
    np.testing.assert_allclose(rows, full[tok, hd], rtol=1e-13, atol=1e-14)
    monkeypatch.setattr(oattn, "_ROW_BLOCK", 7)
    blocked = oracle.varlen_attention(q, k, v, cu, 0.25)
    np.testing.assert_allclose(blocked, full, rtol=1e-13, atol=1e-14)


# ---- planted mistakes: each pin above must catch a plausible oracle bug -----

def _planted_transposed(q, k, v, scale, causal=False):
    # contracts over keys with the wrong operand (k and v swapped)
    return oattn.__dict__["_orig_segment_attention"](q, v, k, scale)


def _planted_no_max_subtraction_wrong_axis(q, k, v, scale, causal=False):
    q = np.asarray(q, np.float64); k = np.asarray(k, np.float64); v = np.asarray(v, np.float64)
    out = np.empty_like(q)
    for h in range(q.shape[1]):
        s = q[:, h] @ k[:, h].T * scale
        e = np.exp(s - s.max(0, keepdims=True))
        p = e / e.sum(0, keepdims=True)          # normalised over queries: wrong axis
        out[:, h] = p @ v[:, h]
    return out


def _planted_scale_dropped(q, k, v, scale, causal=False):
    return oattn.__dict__["_orig_segment_attention"](q, k, v, 1.0)


@pytest.mark.parametrize("planted", [_planted_transposed, _planted_no_max_subtraction_wrong_axis,
                                     _planted_scale_dropped])
def test_pins_catch_planted_mistakes(monkeypatch, planted):
    monkeypatch.setitem(oattn.__dict__, "_orig_segment_attention", oattn.segment_attention)
    monkeypatch.setattr(oattn, "segment_attention", planted)
    with pytest.raises(AssertionError):
        test_matches_torch_sdpa_float64([4, 0, 9, 1])


# ---- log-sum-exp of the scores ----------------------------------------------

def _dense_lse_scipy(q, k, cu, scale):
    """scipy's logsumexp over each row of the block-masked score matrix."""
    from scipy.special import logsumexp
    q = np.asarray(q, np.float64); k = np.asarray(k, np.float64)
    T, H, _ = q.shape
    seg = np.searchsorted(cu, np.arange(T), side="right") - 1
    same = seg[:, None] == seg[None, :]
    out = np.empty((T, H))
    for h in range(H):
        s = (q[:, h] @ k[:, h].T) * scale
        out[:, h] = logsumexp(np.where(same, s, -np.inf), axis=1)
    return out


@pytest.mark.parametrize("lens", [[5, 1, 17], [30, 0, 2, 64]])
def test_lse_matches_scipy_on_the_dense_mask(lens):
    rng = np.random.default_rng(21)
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k = (rng.standard_normal((cu[-1], 3, 16)) for _ in range(2))
    np.testing.assert_allclose(oracle.varlen_lse(q, k, cu, 0.3), _dense_lse_scipy(q, k, cu, 0.3),
                               rtol=1e-13, atol=1e-13)


def test_lse_closed_forms_and_bounds():
    rng = np.random.default_rng(22)
    q, k = (rng.standard_normal((1, 2, 8)) for _ in range(2))
    # one key: lse is that key's score
    np.testing.assert_allclose(oracle.segment_lse(q, k, 0.7)[0], 0.7 * np.sum(q[0] * k[0], axis=-1),
                               rtol=1e-14)
    q, k = (rng.standard_normal((50, 2, 8)) for _ in range(2))
    # scale 0: every score is 0, so lse = log(len)
    np.testing.assert_allclose(oracle.segment_lse(q, k, 0.0), np.full((50, 2), np.log(50.0)), rtol=1e-14)
    # max <= lse <= max + log(len), and exp(score - lse) sums to one over the keys
    lse = oracle.segment_lse(q, k, 0.4)
    for h in range(2):
        s = (q[:, h] @ k[:, h].T) * 0.4
        assert np.all(lse[:, h] >= s.max(1) - 1e-12) and np.all(lse[:, h] <= s.max(1) + np.log(50) + 1e-12)
        np.testing.assert_allclose(np.exp(s - lse[:, h:h + 1]).sum(1), 1.0, rtol=1e-13)


def test_lse_pins_catch_a_base_2_mistake(monkeypatch):
    real = oracle.segment_lse
    monkeypatch.setattr(oracle, "segment_lse", lambda q, k, scale: real(q, k, scale) / np.log(2.0))
    with pytest.raises(AssertionError):
        test_lse_closed_forms_and_bounds()
