"""Pins the oracle's 32-token blocks ([Inside engines] "PagedAttention":
physical blocks of e.g. 16 or 32 tokens; a block is handed out when the
current one fills, so waste stays under one block).  Reading: a 32-token
block b is the pair of 16-token planes 2b, 2b+1, and readers go through the
expanded table of planes."""
import random

import numpy as np
import pytest

from oracle.allocator import AllocatorModel, AllocError, expand_table, expand_pairs


def test_slot_through_a_32_token_block_equals_slot_through_its_planes():
    rng = np.random.default_rng(5)
    for _ in range(50):
        row = [int(x) for x in rng.permutation(40)[:int(rng.integers(1, 12))]]
        planes = expand_table(row, 32)
        assert len(planes) == 2 * len(row)
        for p in range(32 * len(row)):
            assert row[p // 32] * 32 + p % 32 == planes[p // 16] * 16 + p % 16
    assert expand_table([3, -1, 5], 32) == [6, 7, -1, -1, 10, 11]
    assert expand_table([3, -1, 5], 16) == [3, -1, 5]
    assert expand_pairs([(1, 4), (2, 0)], 32) == [(2, 8), (3, 9), (4, 0), (5, 1)]


def test_growth_at_32_token_boundaries_and_waste_below_one_block():
    m = AllocatorModel(64, 1, 64, block_tokens=32)
    for n in range(1, 400):
        before = len(m.tables[0])
        m.extend([0], 1)
        grew = len(m.tables[0]) - before
        assert grew == (1 if (n - 1) % 32 == 0 else 0)
        assert 0 <= len(m.tables[0]) * 32 - m.lens[0] <= 31
    m.check_invariants()
    with pytest.raises(AllocError):
        AllocatorModel(8, 1, 8, block_tokens=24)


def test_beams_share_32_token_blocks_and_copy_one_block():
    m = AllocatorModel(16, 4, 8, block_tokens=32)
    m.extend([0], 40)                               # one full block and 8 tokens
    for b in (1, 2, 3):
        m.fork(0, b)
    m.extend([1, 2, 3], 1)
    assert len(m.pending) == 3                      # one 32-token block per divergent beam
    assert len(expand_pairs(m.pending, 32)) == 6    # two 16-token planes each
    assert {t[0] for t in m.tables} == {m.tables[0][0]} and m.ref[m.tables[0][0]] == 4
    m.check_invariants()


def test_prefix_match_and_trim_work_in_32_token_blocks():
    m = AllocatorModel(32, 3, 16, block_tokens=32)
    keys = list(range(100))
    m.extend([0], 100)
    m.prefix_commit(0, keys)
    assert len(m.entries) == 3                      # 96 tokens in full 32-token blocks
    assert m.prefix_match(1, keys) == 96
    assert m.prefix_match(2, keys[:40] + [999] + keys[41:]) == 32
    m.free_seq(1)
    m.free_seq(2)
    m.extend([1], 300)
    assert m.trim_window([1], 50) == (300 - 50) // 32
    held = [b for b in m.tables[1] if b >= 0]
    assert len(held) <= -(-50 // 32) + 1
    assert all(b < 0 for b in m.tables[1][:(300 - 50) // 32])
    m.check_invariants()
