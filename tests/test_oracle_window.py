"""Pins the oracle's sliding window ([KV essay] "Capping the window instead
of shrinking the rows"): attention covers a trailing span of W positions,
entries older than the span can be dropped, the cache's size is then
bounded by W, and a 32K context with a 4096-token window needs an eighth of the
memory (0.5 GB instead of 4 GB for the Mistral-7B shape the page prices)."""
import math

import numpy as np
import pytest

from oracle import attention as att
from oracle.allocator import AllocatorModel, AllocError, BLOCK_TOKENS
from oracle.inject import InjectError, validate_runs
from oracle.kv_size import kv_bytes
from oracle.layout import PoolSpec, slot, k_element_offsets, v_element_offsets
from oracle.numerics import f32_to_bf16_rne, to_f64


def filled_pool(rng, lens, H=2, d=64, extra=3):
    need = sum(-(-n // BLOCK_TOKENS) for n in lens)
    nb = need + extra
    spec = PoolSpec(1, nb, H, d, "bf16").resolved()
    kp = f32_to_bf16_rne(rng.standard_normal(spec.elements()).astype(np.float32))
    vp = f32_to_bf16_rne(rng.standard_normal(spec.elements()).astype(np.float32))
    perm = [int(x) for x in rng.permutation(nb)]
    tables, at = [], 0
    for n in lens:
        k = -(-n // BLOCK_TOKENS)
        tables.append(perm[at:at + k])
        at += k
    return spec, kp, vp, tables


def test_window_at_least_the_length_is_full_attention():
    rng = np.random.default_rng(1)
    lens = [1, 17, 40, 100]
    spec, kp, vp, tables = filled_pool(rng, lens)
    q = f32_to_bf16_rne(rng.standard_normal((4, 4, 64)).astype(np.float32))
    full = att.decode_paged(q, kp, vp, spec, 0, tables, lens, 4)
    for w in (100, 101, 10 ** 6):
        got = att.decode_paged(q, kp, vp, spec, 0, tables, lens, 4, window=w)
        assert np.array_equal(got[0], full[0]) and np.array_equal(got[1], full[1])


def test_window_of_one_returns_the_last_value():
    rng = np.random.default_rng(2)
    lens = [5, 33, 64]
    spec, kp, vp, tables = filled_pool(rng, lens)
    q = f32_to_bf16_rne(rng.standard_normal((3, 4, 64)).astype(np.float32))
    out, lse = att.decode_paged(q, kp, vp, spec, 0, tables, lens, 4, window=1)
    for b, n in enumerate(lens):
        blk, t = divmod(slot(tables[b], n - 1), BLOCK_TOKENS)
        for h in range(4):
            v = to_f64(vp[v_element_offsets(spec, 0, blk, h // 2, t)], "bf16")
            k = to_f64(kp[k_element_offsets(spec, 0, blk, h // 2, t)], "bf16")
            assert np.array_equal(out[b, h], v)
            assert lse[b, h] == pytest.approx(float(k @ to_f64(q[b, h], "bf16")) / 8.0, abs=1e-12)


def test_windowed_paged_decode_is_attention_over_the_last_w_positions():
    rng = np.random.default_rng(3)
    lens = [30, 47, 129, 200]
    spec, kp, vp, tables = filled_pool(rng, lens)
    q = f32_to_bf16_rne(rng.standard_normal((4, 4, 64)).astype(np.float32))
    for w in (2, 15, 16, 17, 33, 64):
        out, lse = att.decode_paged(q, kp, vp, spec, 0, tables, lens, 4, window=w)
        for b, n in enumerate(lens):
            lo = max(0, n - w)
            ks, vs = [], []
            for p in range(lo, n):
                blk, t = divmod(slot(tables[b], p), BLOCK_TOKENS)
                ks.append([to_f64(kp[k_element_offsets(spec, 0, blk, h, t)], "bf16") for h in range(2)])
                vs.append([to_f64(vp[v_element_offsets(spec, 0, blk, h, t)], "bf16") for h in range(2)])
            ks, vs = np.array(ks), np.array(vs)
            for h in range(4):
                qh = to_f64(q[b, h], "bf16")
                s = ks[:, h // 2, :] @ qh / 8.0
                m = s.max()
                wgt = np.exp(s - m)
                ref = wgt @ vs[:, h // 2, :] / wgt.sum()
                assert np.allclose(out[b, h], ref, rtol=0, atol=1e-12)
                assert lse[b, h] == pytest.approx(m + math.log(wgt.sum()), abs=1e-12)


def test_trim_keeps_exactly_the_window_mistral_numbers():
    # Mistral-7B shape as the page prices it: 32 layers, 8 KV heads, d=128,
    # fp16; 32K context costs 4 GB, a 4096-token window 0.5 GB.
    L, H, d, ctx, W = 32, 8, 128, 32768, 4096
    m = AllocatorModel(4096, 1, 4096)
    m.extend([0], ctx)
    assert m.trim_window([0], W) == (ctx - W) // BLOCK_TOKENS
    held = [b for b in m.tables[0] if b >= 0]
    assert len(held) * BLOCK_TOKENS == W
    assert kv_bytes(L, H, d, 2, ctx) == 4 * 2 ** 30
    assert kv_bytes(L, H, d, 2, len(held) * BLOCK_TOKENS) == 2 ** 29
    assert kv_bytes(L, H, d, 2, ctx) // kv_bytes(L, H, d, 2, len(held) * BLOCK_TOKENS) == 8
    m.check_invariants()


def test_cache_size_is_bounded_by_the_window():
    W = 50
    m = AllocatorModel(64, 2, 64)
    held = []
    for n in range(1, 400):
        m.extend([0], 1)
        m.trim_window([0], W)
        held.append(sum(1 for b in m.tables[0] if b >= 0))
        # the blocks hold the last W positions and at most one partial block more
        assert held[-1] <= -(-W // BLOCK_TOKENS) + 1
        first = next(i for i, b in enumerate(m.tables[0]) if b >= 0)
        assert first * BLOCK_TOKENS <= max(0, n - W)
    assert max(held) == -(-W // BLOCK_TOKENS) + 1 and len(m.free) >= 64 - max(held)
    m.check_invariants()


def test_trim_respects_sharing_and_rejects_writes_into_dropped_blocks():
    m = AllocatorModel(32, 3, 16)
    m.extend([0], 100)
    m.fork(0, 1)
    blocks = list(m.tables[0])
    m.trim_window([0], 20)                      # drops blocks 0..4 of seq 0 only
    assert m.tables[0][:5] == [-1] * 5 and m.tables[1] == blocks
    assert all(m.ref[b] == 1 for b in blocks[:5]) and not set(blocks[:5]) & set(m.free)
    m.trim_window([1], 20)
    assert set(blocks[:5]) <= set(m.free)
    with pytest.raises(AllocError) as e:
        m.prepare_inject([(0, 4, 10, 0)])
    assert e.value.code == "RANGE"
    with pytest.raises(InjectError) as e:
        validate_runs(m.tables, m.lens, [(0, 4, 10, 0)], 1000)
    assert e.value.code == "RANGE"
    with pytest.raises(AllocError) as e:
        m.prefix_commit(0, list(range(32)))
    assert e.value.code == "RANGE"
    with pytest.raises(AllocError) as e:
        m.trim_window([0], 0)
    assert e.value.code == "INVALID"
    m.free_seq(0)
    m.free_seq(1)
    assert len(m.free) == 32
    m.check_invariants()
