"""Pins for the oracle's storage rounding to float32 and its dtype dispatch.

``_RMSNorm.forward`` on the vLLM page casts its result back to the input dtype;
the oracle models that as one round-to-nearest-even of the exact value
(``oracle.rounding``).  ``round_to_bf16`` is pinned in ``test_oracle_prepass``;
here:

* ``round_to_f32``: hand cases at float32's 24-bit significand (ties to even
  in both directions, a value just past a tie, large and negative values,
  values that are already float32), and agreement with an independent
  significand rounding written from the definition (``frexp`` / ``rint`` /
  ``ldexp`` at 24 bits) on 10^5 random fp64 values;
* ``round_to_dtype``: "bf16" reaches the 8-bit rounding and "f32" the 24-bit
  one (checked on values where the two differ), anything else raises
  ``ValueError``;
* planted mistakes (the dispatch swapped, a rounding that returns its input)
  must fail these pins.
"""
import numpy as np
import pytest

import oracle
from oracle import rounding as orounding


def _round_significand(x, bits):
    """Round-to-nearest-even keeping ``bits`` significant bits (normal range)."""
    m, e = np.frexp(np.asarray(x, dtype=np.float64))
    return np.ldexp(np.rint(np.ldexp(m, bits)), e - bits)


def test_f32_rounding_hand_cases():
    r = oracle.round_to_f32
    u = 2.0 ** -23                                                   # float32 ulp at 1
    assert r(np.float64(1.0 + u / 2)) == 1.0                         # tie -> even (down)
    assert r(np.float64(1.0 + 3 * u / 2)) == 1.0 + 2 * u             # tie -> even (up)
    assert r(np.float64(1.0 + u / 2 + 2.0 ** -40)) == 1.0 + u        # just past the tie
    assert r(np.float64(1.0 + u / 2 - 2.0 ** -40)) == 1.0            # just before it
    assert r(np.float64(2.0 ** 24 + 1)) == 2.0 ** 24                 # integer tie -> even
    assert r(np.float64(2.0 ** 24 + 3)) == 2.0 ** 24 + 4
    assert r(np.float64(-(2.0 ** 24 + 3))) == -(2.0 ** 24 + 4)       # symmetric in sign
    assert r(np.float64(0.1)) == 13421773 * 2.0 ** -27               # 0.1 to 24 bits
    assert r(np.float64(0.0)) == 0.0
    # already float32 values are returned unchanged: short significands, and
    # the largest float32 (24 ones times 2^104)
    for exact in (1.5, -0.75, 2.0 ** -100, (2.0 ** 24 - 1) * 2.0 ** 104):
        assert r(np.float64(exact)) == exact


def test_f32_rounding_agrees_with_significand_rounding():
    rng = np.random.default_rng(21)
    x = rng.standard_normal(100000) * np.exp2(rng.integers(-40, 40, 100000))
    np.testing.assert_array_equal(oracle.round_to_f32(x), _round_significand(x, 24))


def test_round_to_dtype_dispatch():
    x = np.array([1.0 + 2.0 ** -10, 3.0 + 2.0 ** -20, -0.1])
    # bf16 keeps 8 bits, f32 keeps 24: the two differ on every one of these
    np.testing.assert_array_equal(oracle.round_to_dtype(x, "bf16"), _round_significand(x, 8))
    np.testing.assert_array_equal(oracle.round_to_dtype(x, "f32"), _round_significand(x, 24))
    assert not np.array_equal(oracle.round_to_dtype(x, "bf16"), oracle.round_to_dtype(x, "f32"))
    for bad in ("fp16", "float32", "", "BF16"):
        with pytest.raises(ValueError):
            oracle.round_to_dtype(x, bad)


def _planted_identity(x):
    return np.asarray(x, dtype=np.float64)


@pytest.mark.parametrize("name,fn", [("round_to_f32", orounding.round_to_bf16),
                                     ("round_to_f32", _planted_identity),
                                     ("round_to_bf16", orounding.round_to_f32)])
def test_pins_catch_planted_rounding_mistakes(monkeypatch, name, fn):
    monkeypatch.setattr(orounding, name, fn)
    monkeypatch.setattr(oracle, name, fn)
    failed = 0
    for pin in (test_f32_rounding_hand_cases, test_f32_rounding_agrees_with_significand_rounding,
                test_round_to_dtype_dispatch):
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed >= 1
