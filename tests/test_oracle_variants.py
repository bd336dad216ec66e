"""Pins for the oracle's variants on the pages: the uniform batch
(``cu_seqlens = None``), the causal flag, and complex-form RoPE.

* uniform batch: the boundaries' defining properties (start 0, constant step
  ``seq_len``, end ``bsz * seq_len``); the attention equals batched 4-D
  attention written with whole-tensor matmuls over ``[B, H, S, S]``;
* causal: brute force over the full ``T x T`` score matrix with an additive
  block-diagonal causal mask (the shape of ``VisionAttention.forward`` on the
  vLLM page); a segment's first row is its value row exactly; its last row is
  the non-causal row; the first row's log-sum-exp is its own score;
* complex RoPE: hand-derived values for D = 4 (one pair per axis, turning by
  ``row`` and ``col`` radians); the equivalence with the rotate-half form
  under the interleave permutation; identity at (0, 0); length of every pair;
  the relative-position property.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# ---------------------------------------------------------------- uniform batch

@pytest.mark.parametrize("bsz,s", [(3, 4), (1, 17), (5, 1), (0, 9), (4, 0)])
def test_uniform_cu_seqlens_properties(bsz, s):
    cu = oracle.uniform_cu_seqlens(bsz, s)
    assert cu.dtype == np.int32 and cu.shape == (bsz + 1,)
    assert cu[0] == 0 and cu[-1] == bsz * s
    assert np.all(np.diff(cu) == s)


def test_uniform_cu_seqlens_rejects_negative():
    with pytest.raises(ValueError):
        oracle.uniform_cu_seqlens(-1, 4)


@pytest.mark.parametrize("causal", [False, True])
def test_dense_batch_equals_batched_4d_attention(causal):
    B, S, H, D = 3, 7, 2, 8
    q, k, v = (_rand((B * S, H, D), i) for i in range(3))
    scale = 0.3
    got = oracle.dense_batch_attention(q, k, v, B, S, scale, causal=causal)
    # whole-batch form: [B, H, S, S] scores from one batched matmul
    qb, kb, vb = (torch.from_numpy(x.reshape(B, S, H, D)).permute(0, 2, 1, 3) for x in (q, k, v))
    scores = torch.matmul(qb, kb.transpose(-1, -2).contiguous()) * scale
    if causal:
        scores = scores.masked_fill(torch.triu(torch.ones(S, S, dtype=torch.bool), 1), -math.inf)
    want = torch.matmul(torch.softmax(scores, dim=-1), vb).permute(0, 2, 1, 3).reshape(B * S, H, D)
    np.testing.assert_allclose(got, want.numpy(), rtol=0, atol=1e-13)


# ---------------------------------------------------------------- causal

def _brute_masked(q, k, v, cu, scale, causal):
    """Full [T, T] scores per head plus an additive mask: 0 where the key is in
    the query's segment (and not after it, if causal), -inf elsewhere."""
    T, H, D = q.shape
    mask = np.full((T, T), -np.inf)
    for i in range(len(cu) - 1):
        a, b = int(cu[i]), int(cu[i + 1])
        for r in range(a, b):
            last = r + 1 if causal else b
            mask[r, a:last] = 0.0
    out = np.full((T, H, D), np.nan)
    for h in range(H):
        s = q[:, h, :] @ k[:, h, :].T * scale + mask
        rows = np.isfinite(s).any(axis=1)
        s = s[rows]
        w = np.exp(s - s.max(axis=1, keepdims=True))
        w /= w.sum(axis=1, keepdims=True)
        out[rows, h, :] = w @ v[:, h, :]
    return out


@pytest.mark.parametrize("causal", [False, True])
def test_causal_brute_force(causal):
    cu = np.array([0, 1, 6, 6, 19, 20], dtype=np.int32)
    q, k, v = (_rand((20, 3, 8), 10 + i) for i in range(3))
    got = oracle.varlen_attention(q, k, v, cu, 0.4, causal=causal)
    want = _brute_masked(q, k, v, cu, 0.4, causal)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-13)


def test_causal_first_row_is_value_and_last_row_is_full():
    cu = np.array([0, 9, 30], dtype=np.int32)
    q, k, v = (_rand((30, 2, 16), 20 + i) for i in range(3))
    c = oracle.varlen_attention(q, k, v, cu, 0.25, causal=True)
    f = oracle.varlen_attention(q, k, v, cu, 0.25, causal=False)
    for a, b in ((0, 9), (9, 30)):
        assert np.array_equal(c[a], v[a])            # one key: weight exactly 1
        np.testing.assert_allclose(c[b - 1], f[b - 1], rtol=0, atol=1e-14)
        assert not np.allclose(c[a + 1:b - 1], f[a + 1:b - 1])


def test_causal_lse_of_first_row_is_its_own_score_and_rows_agree():
    cu = np.array([0, 5, 12], dtype=np.int32)
    q, k, v = (_rand((12, 2, 8), 30 + i) for i in range(3))
    lse = oracle.varlen_lse(q, k, cu, 0.5, causal=True)
    for a in (0, 5):
        np.testing.assert_allclose(lse[a], 0.5 * np.einsum("hd,hd->h", q[a], k[a]), rtol=1e-14)
    # row-by-row evaluation agrees with the segment form
    tokens = np.arange(12)
    heads = tokens % 2
    rows = oracle.varlen_attention_rows(q, k, v, cu, 0.5, tokens, heads, causal=True)
    full = oracle.varlen_attention(q, k, v, cu, 0.5, causal=True)
    np.testing.assert_allclose(rows, full[tokens, heads], rtol=0, atol=1e-14)


# ---------------------------------------------------------------- complex RoPE

def test_complex_rope_hand_values_d4():
    # D = 4: inv_freq = [1], so pair (0, 1) turns by `row` radians and (2, 3) by `col`.
    x = np.array([[[1.0, 0.0, 1.0, 0.0]], [[0.0, 2.0, 3.0, -1.0]]])
    pos = np.array([[1, 2], [3, -5]])
    y = oracle.apply_rope_2d_complex(x, pos)
    want0 = [math.cos(1), math.sin(1), math.cos(2), math.sin(2)]
    # (0 + 2i) e^{3i} and (3 - i) e^{-5i}
    z1 = 2j * complex(math.cos(3), math.sin(3))
    z2 = complex(3, -1) * complex(math.cos(-5), math.sin(-5))
    want1 = [z1.real, z1.imag, z2.real, z2.imag]
    np.testing.assert_allclose(y[0, 0], want0, rtol=0, atol=1e-15)
    np.testing.assert_allclose(y[1, 0], want1, rtol=0, atol=1e-14)


@pytest.mark.parametrize("D", [8, 32, 80, 128])
def test_complex_rope_is_rotate_half_under_the_interleave_permutation(D):
    T, H = 11, 3
    x = _rand((T, H, D), D)
    pos = np.random.default_rng(D + 1).integers(0, 64, size=(T, 2))
    # interleaved pair j = (2j, 2j+1) <-> rotate-half pair (j, j + D/2)
    perm = np.concatenate([np.arange(0, D, 2), np.arange(1, D, 2)])
    inv = np.argsort(perm)
    via_neox = oracle.apply_rope_2d(x[..., perm], pos)[..., inv]
    np.testing.assert_allclose(oracle.apply_rope_2d_complex(x, pos), via_neox, rtol=0, atol=1e-12)


def test_complex_rope_identity_lengths_and_relative_position():
    D = 32
    x = _rand((6, 2, D), 5)
    zero = np.zeros((6, 2), dtype=np.int64)
    np.testing.assert_array_equal(oracle.apply_rope_2d_complex(x, zero), x)
    pos = np.random.default_rng(6).integers(0, 100, size=(6, 2))
    y = oracle.apply_rope_2d_complex(x, pos)
    np.testing.assert_allclose(np.hypot(y[..., 0::2], y[..., 1::2]),
                               np.hypot(x[..., 0::2], x[..., 1::2]), rtol=1e-13)
    # <R(p) a, R(p') b> depends only on p - p'
    a, b = _rand((1, 1, D), 7), _rand((1, 1, D), 8)
    p1, p2, shift = np.array([[3, 9]]), np.array([[14, 2]]), np.array([[40, 25]])
    d0 = np.sum(oracle.apply_rope_2d_complex(a, p1) * oracle.apply_rope_2d_complex(b, p2))
    d1 = np.sum(oracle.apply_rope_2d_complex(a, p1 + shift) * oracle.apply_rope_2d_complex(b, p2 + shift))
    np.testing.assert_allclose(d0, d1, rtol=1e-12)


def test_qk_norm_rope_complex_mode_composes_norm_then_rotation():
    D = 64
    q, k = _rand((5, 2, D), 1), _rand((5, 2, D), 2)
    w = 1 + 0.1 * _rand((D,), 3)
    pos = np.random.default_rng(4).integers(0, 30, size=(5, 2))
    gq, gk = oracle.qk_norm_rope(q, k, pos, 10000.0, w, w, 1e-6, rope_mode="complex")
    tq = torch.nn.functional.rms_norm(torch.from_numpy(q), (D,), torch.from_numpy(w), 1e-6).numpy()
    np.testing.assert_allclose(gq, oracle.apply_rope_2d_complex(tq, pos), rtol=0, atol=1e-12)
    with pytest.raises(ValueError):
        oracle.qk_norm_rope(q, k, pos, rope_mode="gptj")
