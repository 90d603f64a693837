"""Pins the oracle's bfloat16 / float16 rounding against hand-worked values
and a brute-force nearest search over every representable value."""
import numpy as np
import pytest

from oracle.numerics import f32_to_bf16_rne, f32_to_f16_rne, bf16_bits_to_f64, to_f64


def f32(v):
    return np.array([v], dtype=np.float32)


@pytest.mark.parametrize("value,bits", [
    (1.0, 0x3F80),
    (1.0 + 2 ** -8, 0x3F80),            # exact tie -> even (0x3F80)
    (1.0 + 3 * 2 ** -8, 0x3F82),        # exact tie -> even (0x3F82)
    (1.0 + 2 ** -8 + 2 ** -20, 0x3F81),  # just above the tie
    (1.0 + 2 ** -8 - 2 ** -20, 0x3F80),  # just below the tie
    (-1.0 - 3 * 2 ** -8, 0xBF82),
    (0.0, 0x0000),
    (-0.0, 0x8000),
    (np.inf, 0x7F80),
    (-np.inf, 0xFF80),
    (3.4028234663852886e38, 0x7F80),     # beyond max bf16 + half ulp -> inf
    (3.3895313892515355e38, 0x7F7F),     # max finite bf16 stays
    (2 ** -133, 0x0001),                 # smallest bf16 subnormal
])
def test_bf16_hand_worked(value, bits):
    assert int(f32_to_bf16_rne(f32(value))[0]) == bits


def test_bf16_nan_is_quiet():
    out = int(f32_to_bf16_rne(f32(np.nan))[0])
    assert (out & 0x7F80) == 0x7F80 and (out & 0x7F) != 0


def _nearest_even(x64, pos_bits, pos_vals):
    """Brute force: nearest positive finite value to |x|, ties to even bits."""
    ax = abs(x64)
    i = int(np.searchsorted(pos_vals, ax))
    cands = [k for k in (i - 1, i) if 0 <= k < len(pos_vals)]
    dist = [abs(pos_vals[k] - ax) for k in cands]
    best = min(dist)
    win = [int(pos_bits[k]) for k, dd in zip(cands, dist) if dd == best]
    if len(win) > 1:
        win = [w for w in win if w % 2 == 0]
    return win[0] | (0x8000 if x64 < 0 else 0)


def test_bf16_brute_force_nearest():
    pos_bits = np.arange(0, 0x7F80, dtype=np.uint16)       # +0 .. max finite
    pos_vals = bf16_bits_to_f64(pos_bits)
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(5000).astype(np.float32),
                        (rng.standard_normal(500) * 1e-38).astype(np.float32),
                        (rng.standard_normal(500) * 1e30).astype(np.float32)])
    got = f32_to_bf16_rne(x)
    for xi, gi in zip(x.astype(np.float64), got):
        if xi == 0:
            continue
        assert int(gi) == _nearest_even(xi, pos_bits, pos_vals), xi


def test_f16_brute_force_nearest():
    pos_bits = np.arange(0, 0x7C00, dtype=np.uint16)
    pos_vals = pos_bits.view(np.float16).astype(np.float64)
    rng = np.random.default_rng(8)
    x = np.concatenate([rng.standard_normal(5000).astype(np.float32),
                        (rng.standard_normal(500) * 1e-6).astype(np.float32),
                        (rng.standard_normal(500) * 1e4).astype(np.float32)])
    got = f32_to_f16_rne(x)
    for xi, gi in zip(x.astype(np.float64), got):
        if xi == 0:
            continue
        assert int(gi) == _nearest_even(xi, pos_bits, pos_vals), xi


@pytest.mark.parametrize("value,bits", [
    (1.0, 0x3C00),
    (1.0 + 2 ** -11, 0x3C00),            # tie -> even
    (1.0 + 3 * 2 ** -11, 0x3C02),        # tie -> even
    (65504.0, 0x7BFF),
    (65520.0, 0x7C00),                   # tie between max and 2^16 -> inf
    (2 ** -24, 0x0001),
    (2 ** -25, 0x0000),                  # tie with zero -> even (zero)
    (3 * 2 ** -25, 0x0002),              # tie -> even
    (-2.0, 0xC000),
])
def test_f16_hand_worked(value, bits):
    assert int(f32_to_f16_rne(f32(value))[0]) == bits


def test_widening_exact():
    x = np.array([1.5, -2.25, 3.0e-5, 1234.5], dtype=np.float32)
    b = f32_to_bf16_rne(x)
    assert np.array_equal(to_f64(b, "bf16"), np.array([1.5, -2.25, bf16_bits_to_f64(b[2:3])[0], 1232.0]))
    h = f32_to_f16_rne(x)
    assert to_f64(h, "f16")[0] == 1.5 and to_f64(h, "f16")[3] == 1234.0  # tie at ulp 1 -> even
