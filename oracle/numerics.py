"""Element formats of the cache (oracle; test infrastructure only).

The pages fix no rounding rule for storing a rotated key; the reading taken
is IEEE round-to-nearest, ties-to-even, for bfloat16 and float16 alike.  Both
are written here from that definition, not from any bit trick: the bfloat16
rounding picks the nearer of the two bfloat16 neighbours of the float32 value
and breaks a tie towards the even significand.

Storage formats are held as raw integers: bfloat16 and float16 as uint16,
float32 as float32.  Widening to float64 is exact for all three.
"""

import numpy as np

DTYPES = ("f32", "bf16", "f16", "fp8")
ELEM_BYTES = {"f32": 4, "bf16": 2, "f16": 2, "fp8": 1}


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact value of bfloat16 bit patterns (uint16) as float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f16_bits_to_f64(bits) -> np.ndarray:
    """Exact value of IEEE binary16 bit patterns (uint16) as float64."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def to_f64(raw, dtype: str) -> np.ndarray:
    """Widen stored elements of ``dtype`` to float64 (exact; fp8 unscaled)."""
    if dtype == "fp8":
        return e4m3_to_f64(raw)
    if dtype == "f32":
        return np.asarray(raw, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_bits_to_f64(raw)
    if dtype == "f16":
        return f16_bits_to_f64(raw)
    raise ValueError(dtype)


def to_f32(raw, dtype: str) -> np.ndarray:
    """Widen stored elements to float32 (exact for every storage format)."""
    return to_f64(raw, dtype).astype(np.float32)


def _bf16_value(bits32: np.ndarray) -> np.ndarray:
    """float64 value of a float32 bit pattern whose low 16 bits are zero.

    The pattern one past the largest finite bfloat16 (exponent all ones) is
    valued at 2**128, the next value the format would have, so that overflow
    follows the round-to-nearest rule.
    """
    bits32 = bits32.astype(np.uint32)
    exp_all_ones = (bits32 & np.uint32(0x7F800000)) == np.uint32(0x7F800000)
    v = bits32.view(np.float32).astype(np.float64)
    sign = np.where((bits32 >> np.uint32(31)) != 0, -1.0, 1.0)
    return np.where(exp_all_ones, sign * 2.0 ** 128, v)


def f32_to_bf16_rne(x) -> np.ndarray:
    """Round float32 values to bfloat16, nearest with ties to even (uint16).

    For a finite x, ``lo`` is x with its low 16 bits cleared (the bfloat16
    neighbour towards zero) and ``hi`` the next bfloat16 away from zero; the
    nearer wins, a tie goes to the one whose last significand bit is 0.  NaN
    becomes the quiet NaN of the same sign; infinities stay infinite.
    """
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x.view(np.uint32)
    lo = u & np.uint32(0xFFFF0000)
    hi = lo + np.uint32(0x10000)
    xv = x.astype(np.float64)
    d_lo = np.abs(xv - _bf16_value(lo))
    d_hi = np.abs(_bf16_value(hi) - xv)
    lo_even = ((lo >> np.uint32(16)) & np.uint32(1)) == 0
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ~lo_even)
    out = np.where(take_hi, hi, lo) >> np.uint32(16)
    is_nan = np.isnan(x)
    is_inf = np.isinf(x)
    out = np.where(is_inf, u >> np.uint32(16), out)
    out = np.where(is_nan, (u >> np.uint32(16)) & np.uint32(0x8000) | np.uint32(0x7FC0), out)
    return out.astype(np.uint16)


def f32_to_f16_rne(x) -> np.ndarray:
    """Round float32 values to IEEE binary16, nearest-even (uint16 bits).

    numpy's float32 -> float16 cast is the library routine that performs IEEE
    round-to-nearest-even; it is pinned in the tests against hand-worked
    values, ties and subnormals.
    """
    return np.asarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def from_f32(x, dtype: str) -> np.ndarray:
    """Store float32 values in ``dtype`` (identity for f32)."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).copy()
    if dtype == "bf16":
        return f32_to_bf16_rne(x)
    if dtype == "f16":
        return f32_to_f16_rne(x)
    raise ValueError(dtype)


# -- fp8: OCP E4M3 (1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits) --------
# Used by the quantised cache (the int8/int4 paragraph of "Latency Optimization ›
# KV Cache Management" motivates storing K/V in fewer bits).  Finite values
# go up to 448; the all-ones exponent with all-ones mantissa is NaN; there
# are no infinities.  Codes 0..0x7E are the non-negative finite values.

def e4m3_to_f64(bits) -> np.ndarray:
    """Exact value of E4M3 codes (uint8) as float64, from the field definition."""
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = b & 0x7
    normal = np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64))
    sub = np.ldexp(m / 8.0, -6)
    val = np.where(e == 0, sub, normal)
    nan = (e == 0xF) & (m == 0x7)
    return np.where(nan, np.nan, sign * val)


_E4M3_POS = None


def _e4m3_table():
    global _E4M3_POS
    if _E4M3_POS is None:
        codes = np.arange(0, 0x7F, dtype=np.uint8)        # 0 .. 0x7E: +0 .. 448
        _E4M3_POS = (codes, e4m3_to_f64(codes))
    return _E4M3_POS


def f32_to_e4m3_rne_sat(x) -> np.ndarray:
    """Round float32 values to E4M3: the nearest finite code, ties to the even
    code, magnitudes beyond 448 saturate to 448 (reading: the saturating
    conversion); NaN -> 0x7F with the sign.  Brute force over the 127
    non-negative codes."""
    x = np.asarray(x, dtype=np.float32)
    codes, vals = _e4m3_table()
    a = np.abs(x.astype(np.float64)).ravel()
    i = np.clip(np.searchsorted(vals, a), 1, len(vals) - 1)
    lo, hi = i - 1, i
    d_lo = a - vals[lo]
    d_hi = vals[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((codes[hi] & 1) == 0))
    c = np.where(pick_hi, codes[hi], codes[lo])
    c = np.where(a >= vals[-1], codes[-1], c)               # saturate at 448
    c = np.where(a == 0, 0, c)
    neg = (x.ravel() < 0) | ((x.ravel() == 0) & np.signbit(x.ravel()))
    out = (c.astype(np.uint8) | np.where(neg, 0x80, 0).astype(np.uint8)).astype(np.uint8)
    out = np.where(np.isnan(x.ravel()), np.where(np.signbit(x.ravel()), 0xFF, 0x7F), out)
    return out.astype(np.uint8).reshape(x.shape)
