"""Pins the oracle's fp8 (OCP E4M3) cache format: published constants of the
format, hand-worked ties and saturation, round trips of every code, the
half-ulp error bound, and the fp8 inject/decode paths against dequantised
float64 arithmetic."""
import math

import numpy as np
import pytest

from oracle.numerics import e4m3_to_f64, f32_to_e4m3_rne_sat, f32_to_bf16_rne, to_f64
from oracle import attention as att
from oracle.inject import inject
from oracle.layout import PoolSpec, gather_sequence, slot, k_element_offsets, v_element_offsets
from oracle.rope import rope_table, rope_matrix


@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6), (0x38, 1.0),
    (0x39, 1.125), (0x3F, 1.875), (0x40, 2.0), (0x7E, 448.0), (0xFE, -448.0), (0xB8, -1.0),
])
def test_e4m3_published_values(code, value):
    # OCP 8-bit floating point, E4M3: bias 7, max normal 448 = 1.75 * 2^8,
    # min normal 2^-6, min subnormal 2^-9.
    assert e4m3_to_f64(np.array([code], np.uint8))[0] == value


def test_e4m3_nan_and_negative_zero():
    v = e4m3_to_f64(np.array([0x7F, 0xFF, 0x80], np.uint8))
    assert math.isnan(v[0]) and math.isnan(v[1]) and v[2] == 0 and math.copysign(1, v[2]) < 0


@pytest.mark.parametrize("x,code", [
    (2.0 ** -10, 0x00),        # tie between 0 and 2^-9 -> even code 0
    (3 * 2.0 ** -10, 0x02),    # tie between codes 1 and 2 -> 2
    (1.0625, 0x38),            # tie between 1.0 (0x38) and 1.125 (0x39) -> 0x38
    (1.1875, 0x3A),            # tie between 0x39 and 0x3A -> 0x3A
    (1.0626, 0x39),
    (448.0, 0x7E), (464.0, 0x7E), (1.0e9, 0x7E), (-500.0, 0xFE),   # saturation
    (240.0, 0x77), (-0.0, 0x80),
])
def test_e4m3_hand_worked_rounding(x, code):
    assert int(f32_to_e4m3_rne_sat(np.array([x], np.float32))[0]) == code


def test_e4m3_round_trip_every_code_and_error_bound():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    vals = e4m3_to_f64(codes)
    back = f32_to_e4m3_rne_sat(vals.astype(np.float32))
    assert np.array_equal(back, codes)
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(20000) * rng.choice([1e-3, 1.0, 50.0], 20000)).astype(np.float32)
    x = x[np.abs(x) <= 448]
    q = e4m3_to_f64(f32_to_e4m3_rne_sat(x))
    a = np.abs(x.astype(np.float64))
    # half an ulp: 2^-4 relative for normals, 2^-10 absolute for subnormals
    bound = np.where(a >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(a, 1e-30))) - 4), 2.0 ** -10)
    assert np.all(np.abs(q - x) <= bound + 1e-30)
    order = np.argsort(x)
    assert np.all(np.diff(q[order]) >= 0)


def test_fp8_inject_dequantises_to_the_rotated_key():
    d, H, L = 64, 2, 2
    spec = PoolSpec(L, 6, H, d, "fp8").resolved()
    kp = np.zeros(spec.elements(), np.uint8)
    vp = np.zeros(spec.elements(), np.uint8)
    cos_t, sin_t = rope_table(d, 10000.0, 64)
    rng = np.random.default_rng(8)
    src_k = f32_to_bf16_rne(rng.standard_normal((L, 20, H, d)).astype(np.float32))
    src_v = f32_to_bf16_rne(rng.standard_normal((L, 20, H, d)).astype(np.float32))
    k_scale = np.array([[0.02, 0.05], [0.03, 0.01]], np.float32)
    v_scale = np.array([[0.04, 0.02], [0.05, 0.03]], np.float32)
    tables = [[3, 0, -1]]
    inject(kp, vp, spec, tables, [0], [(0, 20, 7, 0)], src_k.ravel(), src_v.ravel(),
           20 * H * d, H * d, 0, L, "pairs", cos_t, sin_t, src_dtype="bf16", k_scale=k_scale,
           v_scale=v_scale)
    for layer in range(L):
        k, v = gather_sequence(kp, vp, spec, layer, tables[0], 27)
        for t in range(20):
            for h in range(H):
                exact_k = rope_matrix(7 + t, d, 10000.0) @ to_f64(src_k[layer, t, h], "bf16")
                got_k = e4m3_to_f64(k[7 + t, h]) * k_scale[layer, h]
                tol = np.maximum(np.abs(exact_k) * 2.0 ** -4, 2.0 ** -10 * k_scale[layer, h]) * 1.01
                assert np.all(np.abs(got_k - exact_k) <= tol + 1e-6)
                got_v = e4m3_to_f64(v[7 + t, h]) * v_scale[layer, h]
                exact_v = to_f64(src_v[layer, t, h], "bf16")
                tol = np.maximum(np.abs(exact_v) * 2.0 ** -4, 2.0 ** -10 * v_scale[layer, h]) * 1.01
                assert np.all(np.abs(got_v - exact_v) <= tol + 1e-9)


def test_fp8_decode_equals_dequantised_contiguous():
    d, H, HQ = 64, 2, 4
    spec = PoolSpec(1, 10, H, d, "fp8").resolved()
    rng = np.random.default_rng(9)
    lens = [5, 33, 70]
    k_scale = np.array([[0.02, 0.04]], np.float32)
    v_scale = np.array([[0.03, 0.05]], np.float32)
    codes_k = [rng.integers(0, 0x7E, size=(n, H, d)).astype(np.uint8) | (rng.integers(0, 2, size=(n, H, d)) * 0x80).astype(np.uint8) for n in lens]
    codes_v = [rng.integers(0, 0x7E, size=(n, H, d)).astype(np.uint8) for n in lens]
    kp = np.zeros(spec.elements(), np.uint8)
    vp = np.zeros(spec.elements(), np.uint8)
    perm = rng.permutation(10)
    tables, at = [], 0
    for b, n in enumerate(lens):
        nb = -(-n // 16)
        tables.append(list(perm[at:at + nb]))
        at += nb
        for p in range(n):
            blk, t = divmod(slot(tables[b], p), 16)
            for h in range(H):
                kp[k_element_offsets(spec, 0, blk, h, t)] = codes_k[b][p, h]
                vp[v_element_offsets(spec, 0, blk, h, t)] = codes_v[b][p, h]
    q = f32_to_bf16_rne(rng.standard_normal((3, HQ, d)).astype(np.float32))
    out, lse = att.decode_paged(q, kp, vp, spec, 0, tables, lens, HQ, q_dtype="bf16",
                                k_scale=k_scale, v_scale=v_scale)
    q64 = to_f64(q, "bf16")
    for b, n in enumerate(lens):
        for h in range(HQ):
            g = h // 2
            k64 = e4m3_to_f64(codes_k[b][:, g]) * float(k_scale[0, g])
            v64 = e4m3_to_f64(codes_v[b][:, g]) * float(v_scale[0, g])
            o, l = att.softmax_attend(q64[b, h], k64, v64, d ** -0.5)
            assert np.allclose(out[b, h], o, rtol=1e-13, atol=1e-15) and abs(lse[b, h] - l) < 1e-12


def test_fp8_per_block_scales():
    """Scales per (layer, block, KV head): decode dequantises each position
    with the scale of the block it lies in (checked against softmax over
    values dequantised position by position); equal scales in every block
    reproduce the per-head result exactly; the stored code of a value is
    e4m3(v / the scale of its destination block); a block copy carries its
    scales."""
    from oracle.inject import append, copy_blocks
    d, H, HQ, NB = 64, 2, 4, 10
    spec = PoolSpec(1, NB, H, d, "fp8").resolved()
    rng = np.random.default_rng(19)
    lens = [5, 33, 70]
    kb = rng.uniform(0.01, 0.05, size=(1, NB, H)).astype(np.float32)
    vb = rng.uniform(0.01, 0.05, size=(1, NB, H)).astype(np.float32)
    codes_k = [rng.integers(0, 0x7E, size=(n, H, d)).astype(np.uint8) for n in lens]
    codes_v = [rng.integers(0, 0x7E, size=(n, H, d)).astype(np.uint8) for n in lens]
    kp = np.zeros(spec.elements(), np.uint8)
    vp = np.zeros(spec.elements(), np.uint8)
    perm = rng.permutation(NB)
    tables, at = [], 0
    for b, n in enumerate(lens):
        nb = -(-n // 16)
        tables.append(list(perm[at:at + nb]))
        at += nb
        for p in range(n):
            blk, t = divmod(slot(tables[b], p), 16)
            for h in range(H):
                kp[k_element_offsets(spec, 0, blk, h, t)] = codes_k[b][p, h]
                vp[v_element_offsets(spec, 0, blk, h, t)] = codes_v[b][p, h]
    q = f32_to_bf16_rne(rng.standard_normal((3, HQ, d)).astype(np.float32))
    out, lse = att.decode_paged(q, kp, vp, spec, 0, tables, lens, HQ, q_dtype="bf16",
                                k_scale=kb, v_scale=vb)
    q64 = to_f64(q, "bf16")
    for b, n in enumerate(lens):
        blk_of = [int(tables[b][p // 16]) for p in range(n)]
        for h in range(HQ):
            g = h // 2
            k64 = np.stack([e4m3_to_f64(codes_k[b][p, g]) * float(kb[0, blk_of[p], g])
                            for p in range(n)])
            v64 = np.stack([e4m3_to_f64(codes_v[b][p, g]) * float(vb[0, blk_of[p], g])
                            for p in range(n)])
            o, l = att.softmax_attend(q64[b, h], k64, v64, d ** -0.5)
            assert np.allclose(out[b, h], o, rtol=1e-13, atol=1e-15) and abs(lse[b, h] - l) < 1e-12
    # the same scale in every block equals the per-(layer, head) form
    kh = np.array([[0.02, 0.04]], np.float32)
    vh = np.array([[0.03, 0.05]], np.float32)
    o1, l1 = att.decode_paged(q, kp, vp, spec, 0, tables, lens, HQ, q_dtype="bf16",
                              k_scale=kh, v_scale=vh)
    o2, l2 = att.decode_paged(q, kp, vp, spec, 0, tables, lens, HQ, q_dtype="bf16",
                              k_scale=np.repeat(kh[:, None, :], NB, axis=1),
                              v_scale=np.repeat(vh[:, None, :], NB, axis=1))
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    # stored codes use the destination block's scale (no rotation: mode none)
    cos_t, sin_t = rope_table(d, 10000.0, 64)
    ak = np.zeros(spec.elements(), np.uint8)
    av = np.zeros(spec.elements(), np.uint8)
    k_new = f32_to_bf16_rne(rng.standard_normal((1, 2, H, d)).astype(np.float32))
    v_new = f32_to_bf16_rne(rng.standard_normal((1, 2, H, d)).astype(np.float32))
    row = [3, 7]                        # positions 15 and 16: blocks 3 and 7
    append(ak, av, spec, 0, [row], [17], [0], 2, k_new, v_new, "none", cos_t, sin_t,
           src_dtype="bf16", k_scale=kb, v_scale=vb)
    for t, (blk, slot_t) in enumerate([(3, 15), (7, 0)]):
        for h in range(H):
            want_k = f32_to_e4m3_rne_sat(np.divide(to_f64(k_new[0, t, h], "bf16").astype(np.float32),
                                                   kb[0, blk, h], dtype=np.float32))
            want_v = f32_to_e4m3_rne_sat(np.divide(to_f64(v_new[0, t, h], "bf16").astype(np.float32),
                                                   vb[0, blk, h], dtype=np.float32))
            assert np.array_equal(ak[k_element_offsets(spec, 0, blk, h, slot_t)], want_k)
            assert np.array_equal(av[v_element_offsets(spec, 0, blk, h, slot_t)], want_v)
    # a block copy carries the block's scales
    kc, vc = kb.copy(), vb.copy()
    copy_blocks(ak, av, spec, [(3, 9)], k_scale=kc, v_scale=vc)
    assert np.array_equal(kc[:, 9], kb[:, 3]) and np.array_equal(vc[:, 9], vb[:, 3])
    assert np.array_equal(np.delete(kc, 9, axis=1), np.delete(kb, 9, axis=1))
