"""Rotary position embedding at a destination position (oracle; test infra).

[InferScale] §2 (background on positional encoding): RoPE multiplies a query
or key at position p by R_p, a rotation made of 2x2 blocks, and because
R_a^T R_b = R_{b-a} the score of a key rotated to b against a query rotated
to a depends only on b - a.  [InferScale] §3.3 and §5.1: the stored keys
carry no rotation; they are rotated only when composition gives them a
position, with the same cos/sin tables the model uses.

The pages name RoFormer (Su et al.) and nothing more precise.  Readings taken:

* the 2x2 blocks pair dimensions (2i, 2i+1) ("pairs", the literal
  block-diagonal form) or, as a flag, (i, i + d/2) ("halves"); block i turns
  by the angle p * theta_i with theta_i = base ** (-2i/d);
* the rotary table is computed in float64 and rounded once to float32:
  cos_table[p][i] = f32(cos(p * theta_i)), sin_table[p][i] = f32(sin(...)),
  with theta_i from the C library's pow;
* a key is rotated in float32 with no fused multiply-add:
  y0 = f32(f32(x0*c) - f32(x1*s)),  y1 = f32(f32(x0*s) + f32(x1*c)),
  and then stored with round-to-nearest-even (see numerics);
* values are never rotated.
"""

import math

import numpy as np

MODES = ("pairs", "halves", "none")


def thetas(head_dim: int, base: float) -> np.ndarray:
    """theta_i = base ** (-2i/d), i = 0 .. d/2 - 1, in float64.

    Each power is the C library's double-precision pow (Python's math.pow).
    numpy's vectorised power can differ from it in the last bit for some i;
    the reading fixes one float64 function so that the float32 table is a
    single, reproducible rounding of the definition.
    """
    if head_dim % 2:
        raise ValueError("head_dim must be even")
    return np.array([math.pow(float(base), -2.0 * i / head_dim) for i in range(head_dim // 2)],
                    dtype=np.float64)


def rope_rows(head_dim: int, base: float, positions):
    """float32 cos and sin rows of the given positions, shape [n][d/2]."""
    th = thetas(head_dim, base)
    p = np.asarray(positions, dtype=np.float64)[:, None]
    ang = p * th[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def rope_table(head_dim: int, base: float, max_pos: int):
    """float32 cos and sin tables, shape [max_pos][d/2]."""
    return rope_rows(head_dim, base, np.arange(max_pos))


def pair_index(head_dim: int, mode: str):
    """(first, second) dimension index of every 2x2 rotation block."""
    h = head_dim // 2
    if mode == "pairs":
        return np.arange(0, head_dim, 2), np.arange(1, head_dim, 2)
    if mode == "halves":
        return np.arange(h), np.arange(h, head_dim)
    raise ValueError(mode)


def rotate_f32(x, pos, cos_t, sin_t, mode: str) -> np.ndarray:
    """Rotate float32 vectors x[..., d] to positions ``pos`` (broadcast over ...).

    Each 2x2 block is applied as two float32 products and one float32 add or
    subtract, in that order, with every intermediate rounded to float32.
    Mode "none" returns x unchanged.
    """
    x = np.asarray(x, dtype=np.float32)
    if mode == "none":
        return x.copy()
    d = x.shape[-1]
    i0, i1 = pair_index(d, mode)
    pos = np.asarray(pos)
    c = cos_t[pos].astype(np.float32)          # [..., d/2]
    s = sin_t[pos].astype(np.float32)
    x0 = x[..., i0]
    x1 = x[..., i1]
    y = np.empty_like(x)
    a = np.multiply(x0, c, dtype=np.float32)
    b = np.multiply(x1, s, dtype=np.float32)
    y[..., i0] = np.subtract(a, b, dtype=np.float32)
    a = np.multiply(x0, s, dtype=np.float32)
    b = np.multiply(x1, c, dtype=np.float32)
    y[..., i1] = np.add(a, b, dtype=np.float32)
    return y


def rope_matrix(p: float, head_dim: int, base: float, mode: str = "pairs") -> np.ndarray:
    """R_p as a dense float64 matrix (exact-arithmetic reference for tests)."""
    th = thetas(head_dim, base)
    i0, i1 = pair_index(head_dim, mode)
    r = np.zeros((head_dim, head_dim))
    ang = p * th
    c, s = np.cos(ang), np.sin(ang)
    r[i0, i0] = c
    r[i0, i1] = -s
    r[i1, i0] = s
    r[i1, i1] = c
    return r
