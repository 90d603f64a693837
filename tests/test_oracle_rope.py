"""Pins the rotary oracle: the relative-position identity, R_0 = I, a
hand-worked rotation, agreement with the exact matrix, and the two pairings."""
import math

import numpy as np
import pytest

from oracle.rope import rope_table, rotate_f32, rope_matrix, thetas, pair_index


@pytest.mark.parametrize("mode", ["pairs", "halves"])
@pytest.mark.parametrize("d", [2, 64, 128])
def test_relative_identity(mode, d):
    # R_a^T R_b = R_{b-a}, hence <R_a q, R_b k> = <q, R_{b-a} k>
    # (InferScale, background on RoPE in §2).
    rng = np.random.default_rng(d)
    for a, b in [(0, 0), (3, 11), (40, 7), (1000, 4095), (8191, 0)]:
        ra, rb = rope_matrix(a, d, 10000.0, mode), rope_matrix(b, d, 10000.0, mode)
        assert np.allclose(ra.T @ rb, rope_matrix(b - a, d, 10000.0, mode), atol=1e-12)
        q, k = rng.standard_normal(d), rng.standard_normal(d)
        assert abs((ra @ q) @ (rb @ k) - q @ (rope_matrix(b - a, d, 10000.0, mode) @ k)) < 1e-9
        assert np.allclose(ra @ rb, rope_matrix(a + b, d, 10000.0, mode), atol=1e-12)


def test_thetas_closed_form():
    assert np.allclose(thetas(4, 10000.0), [1.0, 0.01])
    th = thetas(128, 10000.0)
    assert th[0] == 1.0 and abs(th[-1] - 10000.0 ** (-126 / 128)) < 1e-18


def test_position_zero_is_identity_bitwise():
    cos_t, sin_t = rope_table(64, 10000.0, 4)
    assert np.all(cos_t[0] == 1.0) and np.all(sin_t[0] == 0.0)
    x = np.random.default_rng(0).standard_normal((5, 64)).astype(np.float32)
    for mode in ("pairs", "halves"):
        assert np.array_equal(rotate_f32(x, np.zeros(5, int), cos_t, sin_t, mode).view(np.uint32),
                              x.view(np.uint32))


def test_hand_worked_quarter_and_unit_angle():
    # d = 2, theta_0 = 1: position 1 turns (1, 0) by one radian, counter-clockwise.
    cos_t, sin_t = rope_table(2, 10000.0, 2)
    y = rotate_f32(np.array([[1.0, 0.0]], np.float32), np.array([1]), cos_t, sin_t, "pairs")
    assert abs(y[0, 0] - 0.5403023058681398) < 1e-7
    assert abs(y[0, 1] - 0.8414709848078965) < 1e-7
    y = rotate_f32(np.array([[0.0, 1.0]], np.float32), np.array([1]), cos_t, sin_t, "pairs")
    assert abs(y[0, 0] + 0.8414709848078965) < 1e-7
    assert abs(y[0, 1] - 0.5403023058681398) < 1e-7


@pytest.mark.parametrize("mode", ["pairs", "halves"])
def test_rotate_matches_exact_matrix(mode):
    d, max_pos = 128, 4096
    cos_t, sin_t = rope_table(d, 10000.0, max_pos)
    rng = np.random.default_rng(1)
    x = rng.standard_normal((64, d)).astype(np.float32)
    pos = rng.integers(0, max_pos, size=64)
    y = rotate_f32(x, pos, cos_t, sin_t, mode).astype(np.float64)
    for i in range(64):
        exact = rope_matrix(float(pos[i]), d, 10000.0, mode) @ x[i].astype(np.float64)
        # float32 table (1/2 ulp each), two products and one sum: a few 1e-7 relative
        assert np.max(np.abs(y[i] - exact)) < 4e-6 * max(1.0, np.max(np.abs(x[i])))
        assert abs(np.linalg.norm(y[i]) - np.linalg.norm(x[i])) < 1e-5 * np.linalg.norm(x[i])


def test_halves_equals_pairs_under_permutation():
    d = 64
    cos_t, sin_t = rope_table(d, 10000.0, 100)
    rng = np.random.default_rng(2)
    x = rng.standard_normal((10, d)).astype(np.float32)
    pos = rng.integers(0, 100, size=10)
    i0, i1 = pair_index(d, "halves")
    perm = np.empty(d, int)
    perm[0::2], perm[1::2] = i0, i1          # halves layout -> pairs layout
    y_h = rotate_f32(x, pos, cos_t, sin_t, "halves")
    y_p = rotate_f32(x[:, perm], pos, cos_t, sin_t, "pairs")
    assert np.array_equal(y_h[:, perm], y_p)


def test_table_is_fp64_rounded_once():
    cos_t, sin_t = rope_table(128, 10000.0, 300)
    th = [math.pow(10000.0, -2.0 * i / 128) for i in range(64)]
    for p in (1, 17, 299):
        assert np.array_equal(cos_t[p], np.float32([math.cos(p * t) for t in th]))
        assert np.array_equal(sin_t[p], np.float32([math.sin(p * t) for t in th]))


def test_none_mode_is_copy():
    cos_t, sin_t = rope_table(8, 10000.0, 10)
    x = np.arange(16, dtype=np.float32).reshape(2, 8)
    assert np.array_equal(rotate_f32(x, np.array([3, 9]), cos_t, sin_t, "none"), x)
