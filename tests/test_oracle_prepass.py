"""Pins for the oracle's Q/K RMSNorm + 2D rotary pre-pass and its storage rounding.

* frequency table: closed form (theta = 10000, D = 32 gives 10**(-j/2));
* rotary: identity at (0, 0); every rotated pair keeps its length; pair
  (0, D/2) turns by exactly ``row`` radians and pair (D/4, 3D/4) by exactly
  ``col`` radians; the relative-position property; an independent complex-number
  formulation ``(x_m + i x_{m+D/2}) * exp(i a_m)``;
* RMSNorm: PyTorch's ``rms_norm`` in float64 (a library routine), the closed
  form of the mean square with unit weights, scale invariance at eps = 0;
* order: PyTorch ``rms_norm`` then the complex rotation, composed in the order
  ``_qkv_with_rope`` uses on the vLLM page;
* bf16 rounding: hand-checked ties and an independent integer-bit rounding.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import prepass as opre
from vision_encoder_varlen_amd import workloads


def _complex_rope(x, pos, D, theta):
    """Independent rotation: z_m = x_m + i x_{m+D/2} times exp(i a_m)."""
    F = D // 4
    j = np.arange(F, dtype=np.float64)
    inv = theta ** (-4.0 * j / D)   # = 1/theta**(2j/(D/2)) written from the closed form
    ang = np.concatenate([pos[:, :1] * inv[None, :], pos[:, 1:2] * inv[None, :]], axis=1)
    z = x[..., : D // 2] + 1j * x[..., D // 2:]
    z = z * np.exp(1j * ang)[:, None, :]
    return np.concatenate([z.real, z.imag], axis=-1)


def test_inv_freq_closed_form():
    f = oracle.rope_inv_freq(32, 10000.0)
    assert f.shape == (8,)
    np.testing.assert_allclose(f, 10.0 ** (-np.arange(8) / 2.0), rtol=1e-15)
    assert oracle.rope_inv_freq(128)[0] == 1.0
    assert oracle.rope_inv_freq(80).shape == (20,)


def test_rope_identity_at_origin():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((3, 2, 32))
    pos = np.zeros((3, 2), dtype=np.int32)
    assert np.array_equal(oracle.apply_rope_2d(x, pos), x)


@pytest.mark.parametrize("D", [32, 64, 80, 128])
def test_rope_pairs_keep_their_length(D):
    rng = np.random.default_rng(D)
    x = rng.standard_normal((20, 3, D))
    pos = rng.integers(0, 64, size=(20, 2))
    y = oracle.apply_rope_2d(x, pos)
    h = D // 2
    np.testing.assert_allclose(np.hypot(y[..., :h], y[..., h:]), np.hypot(x[..., :h], x[..., h:]),
                               rtol=1e-13)


def test_first_pairs_turn_by_row_and_col_radians():
    D = 64
    rng = np.random.default_rng(1)
    x = rng.standard_normal((1, 1, D))
    row, col = 5, 3
    y = oracle.apply_rope_2d(x, np.array([[row, col]]))
    h, F = D // 2, D // 4
    assert math.isclose(y[0, 0, 0], x[0, 0, 0] * math.cos(row) - x[0, 0, h] * math.sin(row), rel_tol=1e-14)
    assert math.isclose(y[0, 0, h], x[0, 0, h] * math.cos(row) + x[0, 0, 0] * math.sin(row), rel_tol=1e-14)
    assert math.isclose(y[0, 0, F], x[0, 0, F] * math.cos(col) - x[0, 0, h + F] * math.sin(col), rel_tol=1e-14)
    assert math.isclose(y[0, 0, h + F], x[0, 0, h + F] * math.cos(col) + x[0, 0, F] * math.sin(col),
                        rel_tol=1e-14)


@pytest.mark.parametrize("D", [32, 80, 128])
def test_rope_matches_complex_rotation(D):
    rng = np.random.default_rng(2 + D)
    x = rng.standard_normal((50, 2, D))
    pos = rng.integers(0, 128, size=(50, 2))
    np.testing.assert_allclose(oracle.apply_rope_2d(x, pos, 10000.0), _complex_rope(x, pos, D, 10000.0),
                               rtol=1e-12, atol=1e-12)


def test_rope_relative_position_property():
    D = 64
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 1, D))
    k = rng.standard_normal((1, 1, D))
    p1, p2 = np.array([[4, 9]]), np.array([[1, 2]])
    base = float(np.sum(oracle.apply_rope_2d(q, p1) * oracle.apply_rope_2d(k, p2)))
    for shift in ([3, 0], [0, 5], [7, 11]):
        s = np.array([shift])
        moved = float(np.sum(oracle.apply_rope_2d(q, p1 + s) * oracle.apply_rope_2d(k, p2 + s)))
        assert math.isclose(moved, base, rel_tol=1e-11, abs_tol=1e-12)


def test_rms_norm_matches_torch_float64():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((10, 3, 80)) * 3.0
    w = 1 + 0.1 * rng.standard_normal(80)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (80,), torch.from_numpy(w), 1e-6).numpy()
    np.testing.assert_allclose(oracle.rms_norm(x, w, 1e-6), ref, rtol=1e-13, atol=1e-14)


def test_rms_norm_closed_forms():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((7, 2, 64))
    eps = 0.25
    y = oracle.rms_norm(x, np.ones(64), eps)
    msx = np.mean(x * x, -1)
    np.testing.assert_allclose(np.mean(y * y, -1), msx / (msx + eps), rtol=1e-13)
    y1 = oracle.rms_norm(x, np.ones(64), 0.0)
    y2 = oracle.rms_norm(17.5 * x, np.ones(64), 0.0)
    np.testing.assert_allclose(y1, y2, rtol=1e-13)


def test_norm_then_rope_order_and_composition():
    rng = np.random.default_rng(6)
    D = 128
    q = rng.standard_normal((30, 4, D))
    k = rng.standard_normal((30, 4, D))
    wq = 1 + 0.1 * rng.standard_normal(D)
    wk = 1 + 0.1 * rng.standard_normal(D)
    pos = rng.integers(0, 64, size=(30, 2))
    got_q, got_k = oracle.qk_norm_rope(q, k, pos, 10000.0, wq, wk, 1e-6)
    tq = torch.nn.functional.rms_norm(torch.from_numpy(q), (D,), torch.from_numpy(wq), 1e-6).numpy()
    tk = torch.nn.functional.rms_norm(torch.from_numpy(k), (D,), torch.from_numpy(wk), 1e-6).numpy()
    np.testing.assert_allclose(got_q, _complex_rope(tq, pos, D, 10000.0), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(got_k, _complex_rope(tk, pos, D, 10000.0), rtol=1e-11, atol=1e-12)
    # rotary-then-norm differs when the weights are not uniform
    swapped = oracle.rms_norm(oracle.apply_rope_2d(q, pos), wq, 1e-6)
    assert not np.allclose(swapped, got_q, atol=1e-6)


def test_prepass_without_rope_or_norm_is_identity():
    rng = np.random.default_rng(7)
    q = rng.standard_normal((5, 2, 32))
    k = rng.standard_normal((5, 2, 32))
    a, b = oracle.qk_norm_rope(q, k, None)
    assert np.array_equal(a, q) and np.array_equal(b, k)


def test_bf16_rounding_hand_cases():
    r = oracle.round_to_bf16
    assert r(np.float64(1.0 + 2.0 ** -8)) == 1.0                    # tie -> even (down)
    assert r(np.float64(1.0 + 3 * 2.0 ** -8)) == 1.0 + 2.0 ** -6    # tie -> even (up)
    assert r(np.float64(1.0 + 2.0 ** -8 + 2.0 ** -30)) == 1.0 + 2.0 ** -7
    assert r(np.float64(-3.0)) == -3.0
    assert r(np.float64(0.0)) == 0.0
    assert r(np.float64(1000.7)) == 1000.0                          # ulp at 2**9 is 4 -> 1000
    assert r(np.float64(1002.1)) == 1004.0


def test_bf16_rounding_agrees_with_independent_bit_rounding():
    rng = np.random.default_rng(8)
    x = (rng.standard_normal(100000) * 10).astype(np.float32)
    bits = workloads.f32_to_bf16_bits(x)
    via_bits = workloads.bf16_bits_to_f32(bits).astype(np.float64)
    np.testing.assert_array_equal(oracle.round_to_bf16(x.astype(np.float64)), via_bits)


# ---- planted mistakes -------------------------------------------------------

def _planted_col_row_swap(pos, D, theta=10000.0):
    return _orig_angles(np.asarray(pos)[:, ::-1], D, theta)


def _planted_interleaved_freqs(D, theta=10000.0):
    dim = D // 2
    return 1.0 / (float(theta) ** (np.arange(0, dim, 2, dtype=np.float64) / D))  # wrong denominator


def _planted_rotate_sign(x):
    half = x.shape[-1] // 2
    return np.concatenate([x[..., half:], -x[..., :half]], axis=-1)   # rotation the wrong way


_orig_angles = opre.rope_angles


@pytest.mark.parametrize("name,fn", [("rope_angles", _planted_col_row_swap),
                                     ("rope_inv_freq", _planted_interleaved_freqs),
                                     ("_rotate_half", _planted_rotate_sign)])
def test_pins_catch_planted_rope_mistakes(monkeypatch, name, fn):
    monkeypatch.setattr(opre, name, fn)
    failed = 0
    for pin in (test_first_pairs_turn_by_row_and_col_radians, test_inv_freq_closed_form,
                lambda: test_rope_matches_complex_rotation(80)):
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed >= 1
