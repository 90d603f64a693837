"""Pins the oracle's inject/append and decode attention: closed forms,
brute force against a pure-Python softmax, the split-K merge identity,
paged == contiguous, and Theorem 1 (relocated keys give the relative score)."""
import math

import numpy as np
import pytest

from oracle import attention as att
from oracle.inject import inject, append, InjectError, validate_runs
from oracle.layout import PoolSpec, gather_sequence, slot
from oracle.numerics import to_f64, from_f32, f32_to_bf16_rne
from oracle.rope import rope_table, rotate_f32, rope_matrix


def empty_pool(spec):
    return (np.zeros(spec.elements(), spec.storage_dtype()),
            np.zeros(spec.elements(), spec.storage_dtype()))


def py_softmax_attend(q, ks, vs, scale):
    """Pure-Python loops: the textbook formula, no numpy reductions."""
    s = [sum(qi * ki for qi, ki in zip(q, k)) * scale for k in ks]
    m = max(s)
    w = [math.exp(x - m) for x in s]
    l = sum(w)
    out = [sum(w[t] * vs[t][j] for t in range(len(vs))) / l for j in range(len(q))]
    return out, m + math.log(l)


# -- decode closed forms ------------------------------------------------------------
def test_single_token_returns_its_value():
    rng = np.random.default_rng(0)
    q, k, v = rng.standard_normal(64), rng.standard_normal((1, 64)), rng.standard_normal((1, 64))
    out, lse = att.softmax_attend(q, k, v, 0.125)
    assert np.array_equal(out, v[0]) and lse == (k[0] @ q) * 0.125


def test_zero_query_and_equal_keys_give_mean_value():
    rng = np.random.default_rng(1)
    k, v = rng.standard_normal((9, 16)), rng.standard_normal((9, 16))
    out, lse = att.softmax_attend(np.zeros(16), k, v, 0.25)
    assert np.allclose(out, v.mean(0), atol=1e-15) and abs(lse - math.log(9)) < 1e-15
    k_eq = np.tile(rng.standard_normal(16), (9, 1))
    q = rng.standard_normal(16)
    out, _ = att.softmax_attend(q, k_eq, v, 0.25)
    assert np.allclose(out, v.mean(0), atol=1e-14)


def test_two_tokens_sigmoid_form():
    rng = np.random.default_rng(2)
    q, k, v = rng.standard_normal(8), rng.standard_normal((2, 8)), rng.standard_normal((2, 8))
    s1, s2 = (k @ q) * 0.5
    sig = lambda z: 1 / (1 + math.exp(-z))
    out, lse = att.softmax_attend(q, k, v, 0.5)
    assert np.allclose(out, sig(s1 - s2) * v[0] + sig(s2 - s1) * v[1], atol=1e-14)
    assert abs(lse - math.log(math.exp(s1) + math.exp(s2))) < 1e-13


def test_brute_force_every_length_to_48():
    rng = np.random.default_rng(3)
    d = 16
    for n in range(1, 49):
        q, k, v = rng.standard_normal(d), rng.standard_normal((n, d)), rng.standard_normal((n, d))
        out, lse = att.softmax_attend(q, k, v, 1 / math.sqrt(d))
        ref, ref_lse = py_softmax_attend(list(q), k.tolist(), v.tolist(), 1 / math.sqrt(d))
        assert np.allclose(out, ref, rtol=1e-12, atol=1e-13) and abs(lse - ref_lse) < 1e-12


@pytest.mark.parametrize("sizes", [[5], [16, 16, 5], [1, 1, 1], [64, 3], [7, 30, 11, 2]])
def test_lse_merge_equals_direct(sizes):
    rng = np.random.default_rng(sum(sizes))
    n, d = sum(sizes), 32
    q, k, v = rng.standard_normal(d) * 3, rng.standard_normal((n, d)), rng.standard_normal((n, d))
    direct, lse = att.softmax_attend(q, k, v, 0.2)
    cuts = np.cumsum([0] + sizes)
    parts = [att.partial_state(q, k[a:b], v[a:b], 0.2) for a, b in zip(cuts[:-1], cuts[1:])]
    merged, mlse = att.lse_merge(parts)
    assert np.allclose(merged, direct, rtol=1e-12, atol=1e-14) and abs(mlse - lse) < 1e-12


def small_bf16_values(rng, shape):
    return f32_to_bf16_rne(rng.standard_normal(shape).astype(np.float32))


@pytest.mark.parametrize("hq,hkv", [(4, 2), (8, 8), (4, 1), (6, 2)])
def test_paged_equals_contiguous_gqa_mha_mqa(hq, hkv):
    rng = np.random.default_rng(hq * 10 + hkv)
    spec = PoolSpec(1, 24, hkv, 32, "bf16").resolved()
    lens = [1, 15, 16, 17, 33]
    k_seq = [small_bf16_values(rng, (n, hkv, 32)) for n in lens]
    v_seq = [small_bf16_values(rng, (n, hkv, 32)) for n in lens]
    q = small_bf16_values(rng, (len(lens), hq, 32))
    ref, ref_lse = att.decode_contiguous(q, k_seq, v_seq, "bf16", hq)
    from oracle.layout import k_element_offsets, v_element_offsets
    for perm_seed in (0, 1):
        order = np.random.default_rng(perm_seed).permutation(24)
        kp, vp = empty_pool(spec)
        tables, at = [], 0
        for b, n in enumerate(lens):
            nb = -(-n // 16)
            tables.append(list(order[at:at + nb]) + [-1] * (4 - nb))
            at += nb
            for p in range(n):
                blk, t = divmod(slot(tables[b], p), 16)
                for h in range(hkv):
                    kp[k_element_offsets(spec, 0, blk, h, t)] = k_seq[b][p, h]
                    vp[v_element_offsets(spec, 0, blk, h, t)] = v_seq[b][p, h]
        out, lse = att.decode_paged(q, kp, vp, spec, 0, tables, lens, hq)
        assert np.array_equal(out, ref) and np.array_equal(lse, ref_lse)
    # grouped heads: query heads of one group read the same KV head
    g = hq // hkv
    q64 = to_f64(q, "bf16")
    for h in range(hq):
        o, _ = att.softmax_attend(q64[4, h], to_f64(k_seq[4][:, h // g], "bf16"),
                                  to_f64(v_seq[4][:, h // g], "bf16"), 1 / math.sqrt(32))
        assert np.array_equal(o, ref[4, h])


def test_zero_length_sequence():
    spec = PoolSpec(1, 4, 1, 16, "f32").resolved()
    kp, vp = empty_pool(spec)
    q = np.ones((1, 2, 16), np.float32)
    out, lse = att.decode_paged(q, kp, vp, spec, 0, [[-1]], [0], 2)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


def test_out_of_range_block_ids_drop_out_of_attention():
    """Positions whose table entry names no block (negative, or >= num_blocks)
    are left out: the result equals contiguous attention over the remaining
    positions; a sequence with none left gives 0 / -inf."""
    from oracle.layout import k_element_offsets, v_element_offsets
    rng = np.random.default_rng(77)
    nb_pool, hkv, hq, d = 16, 2, 4, 32
    spec = PoolSpec(1, nb_pool, hkv, d, "bf16").resolved()
    lens = [40, 33, 16, 20]
    k_seq = [small_bf16_values(rng, (n, hkv, d)) for n in lens]
    v_seq = [small_bf16_values(rng, (n, hkv, d)) for n in lens]
    q = small_bf16_values(rng, (len(lens), hq, d))
    kp, vp = empty_pool(spec)
    tables, at = [], 0
    for b, n in enumerate(lens):
        nb = -(-n // 16)
        tables.append(list(range(at, at + nb)) + [-1] * (3 - nb))
        at += nb
        for p in range(n):
            blk, t = divmod(slot(tables[b], p), 16)
            for h in range(hkv):
                kp[k_element_offsets(spec, 0, blk, h, t)] = k_seq[b][p, h]
                vp[v_element_offsets(spec, 0, blk, h, t)] = v_seq[b][p, h]
    # seq 0: middle block gone; seq 1: last (partial) block names block 16 =
    # num_blocks; seq 2: its only block is gone; seq 3: first block far out
    tables[0][1] = -1
    tables[1][2] = nb_pool
    tables[2][0] = -(2 ** 31)
    tables[3][0] = 10 ** 6
    kept = [list(range(0, 16)) + list(range(32, 40)), list(range(0, 32)), [],
            list(range(16, 20))]
    ref, ref_lse = att.decode_contiguous(
        q, [k_seq[b][kept[b]] for b in range(4)], [v_seq[b][kept[b]] for b in range(4)],
        "bf16", hq)
    out, lse = att.decode_paged(q, kp, vp, spec, 0, tables, lens, hq, num_blocks=nb_pool)
    assert np.array_equal(out, ref) and np.array_equal(lse, ref_lse)
    assert np.all(out[2] == 0) and np.all(np.isneginf(lse[2]))
    # under a window the same positions drop out of the window's range
    out_w, lse_w = att.decode_paged(q, kp, vp, spec, 0, tables, lens, hq, num_blocks=nb_pool,
                                    window=20)
    kept_w = [[p for p in kept[b] if p >= lens[b] - 20] for b in range(4)]
    ref_w, ref_lse_w = att.decode_contiguous(
        q, [k_seq[b][kept_w[b]] for b in range(4)], [v_seq[b][kept_w[b]] for b in range(4)],
        "bf16", hq)
    assert np.array_equal(out_w, ref_w) and np.array_equal(lse_w, ref_lse_w)


def test_append_skips_out_of_range_block_ids():
    """A token whose table entry names no block is not written; the others are."""
    spec = PoolSpec(1, 6, 2, 64, "bf16").resolved()
    cos_t, sin_t = rope_table(64, 10000.0, 64)
    rng = np.random.default_rng(8)
    k_new = small_bf16_values(rng, (3, 2, 2, 64))
    v_new = small_bf16_values(rng, (3, 2, 2, 64))
    good = [[4, 1, -1], [0, -1, -1], [2, 3, -1]]
    lens_after = [18, 2, 17]          # seq 2's two tokens straddle blocks 2 and 3
    bad = [list(r) for r in good]
    bad[1][0] = 6                      # num_blocks: seq 1 writes nothing
    bad[2][1] = -5                     # seq 2: only its token in block 2 is written
    a_k, a_v = empty_pool(spec)
    append(a_k, a_v, spec, 0, bad, lens_after, [0, 1, 2], 2, k_new, v_new, "pairs", cos_t,
           sin_t, num_blocks=6)
    r_k, r_v = empty_pool(spec)
    append(r_k, r_v, spec, 0, good, lens_after, [0], 2, k_new[0:1], v_new[0:1], "pairs", cos_t,
           sin_t)
    # seq 2, token 0 only (position 15): as an append of one token at length 16
    append(r_k, r_v, spec, 0, good, [0, 0, 16], [2], 1, k_new[2:3, 0:1], v_new[2:3, 0:1],
           "pairs", cos_t, sin_t)
    assert np.array_equal(a_k, r_k) and np.array_equal(a_v, r_v)


def test_append_skips_positions_outside_the_row_and_the_rotary_table():
    """With device-side tables (num_blocks given): tokens at negative
    positions, past the table row or (rotating) at or past max_pos are not
    written; the rest equal a plain append of just those tokens."""
    spec = PoolSpec(1, 8, 1, 32, "bf16").resolved()
    cos_t, sin_t = rope_table(32, 10000.0, 20)            # max_pos 20
    rng = np.random.default_rng(12)
    k_new = small_bf16_values(rng, (3, 4, 1, 32))
    v_new = small_bf16_values(rng, (3, 4, 1, 32))
    tables = [[3, 5], [1, 6], [2, 7]]                    # 32 positions per row
    firsts = [-2, 18, 30]                                # 4 tokens each
    for mode in ("pairs", "none"):
        a_k, a_v = empty_pool(spec)
        append(a_k, a_v, spec, 0, tables, [f + 4 for f in firsts], [0, 1, 2], 4, k_new, v_new,
               mode, cos_t, sin_t, num_blocks=8)
        r_k, r_v = empty_pool(spec)
        # row 0: positions 0, 1 (tokens 2, 3)
        append(r_k, r_v, spec, 0, tables, [2, 0, 0], [0], 2, k_new[0:1, 2:], v_new[0:1, 2:],
               mode, cos_t, sin_t)
        # row 1: 18, 19 rotating; 18..21 without rotation
        n1 = 2 if mode == "pairs" else 4
        append(r_k, r_v, spec, 0, tables, [0, 18 + n1, 0], [1], n1, k_new[1:2, :n1],
               v_new[1:2, :n1], mode, cos_t, sin_t)
        # row 2: 30, 31 without rotation (32, 33 are past the row); none rotating
        if mode == "none":
            append(r_k, r_v, spec, 0, tables, [0, 0, 32], [2], 2, k_new[2:3, :2], v_new[2:3, :2],
                   mode, cos_t, sin_t)
        assert np.array_equal(a_k, r_k) and np.array_equal(a_v, r_v), mode


# -- inject ------------------------------------------------------------------------------
def test_inject_at_position_zero_is_a_bit_copy():
    spec = PoolSpec(1, 2, 2, 64, "bf16").resolved()
    kp, vp = empty_pool(spec)
    cos_t, sin_t = rope_table(64, 10000.0, 64)
    rng = np.random.default_rng(4)
    src_k = small_bf16_values(rng, (1, 1, 2, 64)).ravel()
    src_v = small_bf16_values(rng, (1, 1, 2, 64)).ravel()
    inject(kp, vp, spec, [[1, -1]], [0], [(0, 1, 0, 0)], src_k, src_v, 128, 128, 0, 1,
           "pairs", cos_t, sin_t)
    k, v = gather_sequence(kp, vp, spec, 0, [1], 1)
    assert np.array_equal(k.ravel(), src_k) and np.array_equal(v.ravel(), src_v)


@pytest.mark.parametrize("mode", ["pairs", "halves"])
def test_inject_rotates_to_destination_and_copies_values(mode):
    spec = PoolSpec(2, 8, 2, 64, "bf16").resolved()
    kp, vp = empty_pool(spec)
    cos_t, sin_t = rope_table(64, 10000.0, 128)
    rng = np.random.default_rng(5)
    n_src = 30
    src_k = small_bf16_values(rng, (2, n_src, 2, 64))
    src_v = small_bf16_values(rng, (2, n_src, 2, 64))
    tables = [[5, 2, 7, -1], [0, 3, -1, -1]]
    runs = [(0, 20, 9, 0), (1, 10, 20, 20)]
    lens = inject(kp, vp, spec, tables, [0, 25], runs, src_k.ravel(), src_v.ravel(),
                  n_src * 128, 128, 0, 2, mode, cos_t, sin_t)
    assert lens == [29, 30]
    for layer in range(2):
        for (seq, n, p0, src) in runs:
            k, v = gather_sequence(kp, vp, spec, layer, tables[seq], p0 + n)
            for t in range(n):
                p = p0 + t
                assert np.array_equal(v[p], src_v[layer, src + t])
                exact = np.stack([rope_matrix(p, 64, 10000.0, mode) @ to_f64(src_k[layer, src + t, h], "bf16")
                                  for h in range(2)])
                got = to_f64(k[p], "bf16")
                # bf16 storage: half an ulp (2^-9 relative) plus the float32 rotation error
                assert np.all(np.abs(got - exact) <= 2.0 ** -8 * np.abs(exact) + 1e-6)


def test_inject_validation():
    spec = PoolSpec(1, 4, 1, 16, "f32").resolved()
    kp, vp = empty_pool(spec)
    cos_t, sin_t = rope_table(16, 10000.0, 40)
    src = np.zeros(16 * 100, np.float32)
    tables = [[0, 1, -1], [2, -1, -1]]
    cases = [([(0, 10, 25, 0)], "RANGE"),          # past capacity (32)
             ([(1, 5, 12, 0)], "RANGE"),           # seq 1 capacity 16
             ([(2, 1, 0, 0)], "INVALID"),          # unknown seq
             ([(0, 4, 0, 0), (0, 4, 3, 10)], "OVERLAP"),
             ([(0, 1, 0, -1)], "INVALID")]
    for runs, code in cases:
        with pytest.raises(InjectError) as e:
            inject(kp, vp, spec, tables, [0, 0], runs, src, src, 0, 16, 0, 1, "pairs", cos_t, sin_t)
        assert e.value.code == code
    short_cos, short_sin = rope_table(16, 10000.0, 20)
    with pytest.raises(InjectError) as e:
        inject(kp, vp, spec, tables, [0, 0], [(0, 5, 18, 0)], src, src, 0, 16, 0, 1, "pairs",
               short_cos, short_sin)
    assert e.value.code == "RANGE"
    assert validate_runs(tables, [0, 0], [(0, 0, 31, 0)], 40) == []


def test_inject_empty_runs_write_nothing_and_keep_lengths():
    """An empty run names no position: it writes nothing, is not checked
    against capacity, the rotary table or the store, and leaves the length as
    it is; an unknown sequence or a negative field is still refused."""
    spec = PoolSpec(1, 4, 1, 16, "f32").resolved()
    kp, vp = empty_pool(spec)
    cos_t, sin_t = rope_table(16, 10000.0, 40)
    src = np.arange(16 * 4, dtype=np.float32) + 1.0
    tables = [[0, 1, -1], [2, -1, -1]]
    runs = [(0, 0, 100, 0), (1, 0, 50, 0), (0, 0, 5, 10 ** 6)]
    lens = inject(kp, vp, spec, tables, [3, 0], runs, src, src, 0, 16, 0, 1, "pairs",
                  cos_t, sin_t)
    assert lens == [3, 0]
    assert not kp.any() and not vp.any()
    # beside a run that writes, the length is that run's end alone
    lens = inject(kp, vp, spec, tables, [3, 0], [(0, 2, 4, 0), (0, 0, 30, 0)], src, src, 0,
                  16, 0, 1, "pairs", cos_t, sin_t)
    assert lens == [6, 0]
    for runs, code in (([(2, 0, 0, 0)], "INVALID"), ([(0, 0, -1, 0)], "INVALID"),
                       ([(0, 0, 0, -1)], "INVALID")):
        with pytest.raises(InjectError) as e:
            inject(kp, vp, spec, tables, [0, 0], runs, src, src, 0, 16, 0, 1, "pairs", cos_t,
                   sin_t)
        assert e.value.code == code


def test_append_matches_inject_of_the_same_tokens():
    spec = PoolSpec(1, 6, 2, 64, "bf16").resolved()
    cos_t, sin_t = rope_table(64, 10000.0, 64)
    rng = np.random.default_rng(6)
    k_new = small_bf16_values(rng, (2, 3, 2, 64))
    v_new = small_bf16_values(rng, (2, 3, 2, 64))
    tables = [[4, 1, -1], [0, -1, -1]]
    lens_after = [19, 3]
    a_k, a_v = empty_pool(spec)
    append(a_k, a_v, spec, 0, tables, lens_after, [0, 1], 3, k_new, v_new, "pairs", cos_t, sin_t)
    i_k, i_v = empty_pool(spec)
    runs = [(0, 3, 16, 0), (1, 3, 0, 3)]
    inject(i_k, i_v, spec, tables, [0, 0], runs, k_new.reshape(-1), v_new.reshape(-1),
           0, 128, 0, 1, "pairs", cos_t, sin_t)
    assert np.array_equal(a_k, i_k) and np.array_equal(a_v, i_v)


# -- Theorem 1: relocation gives the prefilled relative scores --------------------------
def test_theorem1_relocated_keys_score_by_relative_position():
    d, n, hq, hkv = 64, 40, 4, 2
    spec = PoolSpec(1, 8, hkv, d, "f32").resolved()
    cos_t, sin_t = rope_table(d, 10000.0, 256)
    rng = np.random.default_rng(7)
    k_pre = rng.standard_normal((1, n, hkv, d)).astype(np.float32)
    v = rng.standard_normal((1, n, hkv, d)).astype(np.float32)
    q_pre = rng.standard_normal((1, hq, d))
    tables = [[6, 1, 3, -1]]
    p0 = 7                                       # chunk placed at positions 7..46
    kp, vp = empty_pool(spec)
    inject(kp, vp, spec, tables, [0], [(0, n, p0, 0)], k_pre.ravel(), v.ravel(),
           0, hkv * d, 0, 1, "pairs", cos_t, sin_t)
    m = 200                                       # the query's own position
    q_rot = np.stack([rope_matrix(m, d, 10000.0) @ q_pre[0, h] for h in range(hq)])[None]
    # keys at positions < p0 are zero in the pool; attend over 7..46 only by
    # comparing against the relative form on the same token set
    k_raw, v_raw = gather_sequence(kp, vp, spec, 0, tables[0], p0 + n)
    g = hq // hkv
    for h in range(hq):
        kk = to_f64(k_raw[p0:, h // g], "f32")
        out, _ = att.softmax_attend(q_rot[0, h], kk, to_f64(v_raw[p0:, h // g], "f32"), d ** -0.5)
        rel_k = np.stack([rope_matrix(p0 + t - m, d, 10000.0) @ k_pre[0, t, h // g].astype(np.float64)
                          for t in range(n)])
        ref, _ = att.softmax_attend(q_pre[0, h], rel_k, v[0, :, h // g].astype(np.float64), d ** -0.5)
        assert np.allclose(out, ref, rtol=1e-5, atol=1e-6)
