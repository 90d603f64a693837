"""Pins the paged layout and the allocator model: the printed block-table
example, on-demand growth, the one-block waste bound, all-or-nothing
reservation, the published splitmix64 vectors, and brute force over short
operation sequences."""
import itertools
import json
import os

import numpy as np
import pytest

from oracle.allocator import (AllocatorModel, AllocError, splitmix64, initial_free_order,
                              BLOCK_TOKENS)
from oracle.layout import (PoolSpec, slot, k_plane_offset, v_plane_offset, gather_sequence,
                           k_element_offsets, v_element_offsets, chunk_elems)
from tests.conftest import GOLDEN


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_worked_block_table_example():
    ex = load("block_table_example.json")
    a = AllocatorModel(ex["num_blocks"], 2, 8)
    a.set_blocks(0, ex["seq_A"]["blocks"], ex["seq_A"]["len"])
    a.set_blocks(1, ex["seq_B"]["blocks"], ex["seq_B"]["len"])
    assert list(a.free)[:len(ex["free_list_prefix"])] == ex["free_list_prefix"]
    assert list(a.free) == ex["free_list_full"]
    for seq, p, s in ex["slot_checks"]:
        assert slot(a.tables[seq], p) == s
    a.extend([1], 13)                         # B: 20 -> 33 needs a third block
    assert a.tables[1][-1] == ex["next_block_allocated"]
    a.check_invariants()


def test_splitmix64_published_vectors():
    ex = load("splitmix64.json")
    g = splitmix64(1234567)
    assert [str(next(g)) for _ in range(5)] == ex["seed_1234567"]
    g = splitmix64(0)
    assert [str(next(g)) for _ in range(3)] == ex["seed_0"]


def test_fisher_yates_direction():
    # The shuffle walks i = N-1 .. 1 and swaps with j = next() mod (i+1).
    ex = load("splitmix64.json")
    v = [int(x) for x in ex["seed_1234567"]]
    order = [0, 1, 2, 3]
    for step, i in enumerate(range(3, 0, -1)):
        j = v[step] % (i + 1)
        order[i], order[j] = order[j], order[i]
    assert initial_free_order(4, 1234567) == order
    big = initial_free_order(1000, 99)
    assert sorted(big) == list(range(1000)) and big != list(range(1000))
    assert initial_free_order(7, 0) == list(range(7))


def test_on_demand_growth_at_block_boundary():
    a = AllocatorModel(64, 1, 64)
    owned = []
    for n in range(1, 200):
        a.extend([0], 1)
        owned.append(len(a.tables[0]))
        assert len(a.tables[0]) == -(-n // 16)
        assert len(a.tables[0]) * 16 - a.lens[0] <= 15     # waste bound
    grew = [n for n in range(1, 199) if owned[n] != owned[n - 1]]
    assert all((n % 16) == 0 for n in grew)               # len went 16k -> 16k+1


def test_oom_is_all_or_nothing():
    a = AllocatorModel(4, 3, 8)
    a.extend([0, 1], 16)
    snap = (list(a.free), [list(t) for t in a.tables], list(a.lens))
    with pytest.raises(AllocError) as e:
        a.extend([0, 1, 2], 17)                # needs 1 + 1 + 2 = 4 > 2 free
    assert e.value.code == "OOM"
    assert (list(a.free), [list(t) for t in a.tables], list(a.lens)) == snap
    with pytest.raises(AllocError) as e:
        a.alloc_blocks(2, 16 * 3)
    assert e.value.code == "OOM"
    assert (list(a.free), [list(t) for t in a.tables], list(a.lens)) == snap


def test_free_returns_blocks_fifo():
    a = AllocatorModel(6, 2, 8)
    a.alloc_blocks(0, 40)                        # 0, 1, 2
    a.alloc_blocks(1, 20)                        # 3, 4
    a.free_seq(0)
    assert list(a.free) == [5, 0, 1, 2]
    a.alloc_blocks(1, 60)                        # + 5, 0
    assert a.tables[1] == [3, 4, 5, 0]


def test_errors():
    a = AllocatorModel(4, 2, 2)
    with pytest.raises(AllocError) as e:
        a.alloc_blocks(5, 1)
    assert e.value.code == "INVALID"
    with pytest.raises(AllocError) as e:
        a.alloc_blocks(0, 33)
    assert e.value.code == "RANGE"
    a.alloc_blocks(0, 1)
    with pytest.raises(AllocError) as e:
        a.set_blocks(1, [0], 1)                  # block 0 is owned
    assert e.value.code == "INVALID"
    with pytest.raises(AllocError) as e:
        a.set_blocks(0, [1], 1)                  # seq 0 not empty
    assert e.value.code == "INVALID"


def test_brute_force_short_op_sequences():
    ops = [("ext", s, n) for s in (0, 1) for n in (1, 15, 17)] + [("free", s, 0) for s in (0, 1)]
    for seq in itertools.product(ops, repeat=4):
        a = AllocatorModel(4, 2, 4)
        for kind, s, n in seq:
            before = (list(a.free), [list(t) for t in a.tables], list(a.lens))
            try:
                if kind == "ext":
                    a.extend([s], n)
                else:
                    a.free_seq(s)
            except AllocError:
                assert (list(a.free), [list(t) for t in a.tables], list(a.lens)) == before
            a.check_invariants()
            for t in range(2):
                assert len(a.tables[t]) == -(-a.lens[t] // 16)


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 128), ("f16", 128), ("bf16", 64)])
def test_plane_offsets_are_bijections(dtype, d):
    t, j = np.meshgrid(np.arange(16), np.arange(d), indexing="ij")
    ko = k_plane_offset(t, j, dtype).ravel()
    vo = v_plane_offset(t, j).ravel()
    assert sorted(ko.tolist()) == list(range(16 * d))
    assert sorted(vo.tolist()) == list(range(16 * d))
    x = chunk_elems(dtype)
    # one K chunk = X consecutive dims of one token, 16 bytes
    assert x * (4 if dtype == "f32" else 2) == 16
    assert np.all(np.diff(k_plane_offset(3, np.arange(x), dtype)) == 1)
    assert np.all(np.diff(v_plane_offset(np.arange(16), 5)) == 1)


def _plane_cases():
    import json
    import os
    from tests.conftest import GOLDEN
    with open(os.path.join(GOLDEN, "plane_offsets.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _plane_cases(), ids=lambda c: "%s-t%d-j%d" % (c["dtype"], c["t"], c["j"]))
def test_plane_offsets_equal_hand_worked_values(case):
    """The oracle's in-plane offsets against values worked by hand from the
    layout the C header states (tests/golden/plane_offsets.json)."""
    assert int(k_plane_offset(case["t"], case["j"], case["dtype"])) == case["k"], case["work"]
    assert int(v_plane_offset(case["t"], case["j"])) == case["v"], case["work"]


def test_plane_offset_pins_reject_plausible_other_layouts():
    """Each plausible misreading of the layout disagrees with some hand-worked
    value: a token-major K plane (all dims of token t together), chunks of the
    wrong width, or a token-major V plane."""
    cases = _plane_cases()
    x = {"f32": 4, "bf16": 8, "f16": 8, "fp8": 16}
    d_of = {"f32": 64, "bf16": 128, "f16": 64, "fp8": 128}

    def token_major_k(t, j, dt):
        return t * d_of[dt] + j

    def wrong_chunk_k(t, j, dt):               # chunks of 8 dims whatever the element size
        return ((j // 8) * 16 + t) * 8 + j % 8

    def token_major_v(t, j, dt):
        return t * d_of[dt] + j

    for name, fk in (("token-major K", token_major_k), ("8-dim chunks", wrong_chunk_k)):
        assert any(fk(c["t"], c["j"], c["dtype"]) != c["k"] for c in cases), name
    assert any(token_major_v(c["t"], c["j"], c["dtype"]) != c["v"] for c in cases)


def test_paged_gather_equals_contiguous_under_any_permutation():
    spec = PoolSpec(2, 12, 2, 64, "bf16").resolved()
    rng = np.random.default_rng(3)
    lens = [37, 100 - 64]
    k_seq = [rng.integers(0, 2 ** 16, size=(n, 2, 64), dtype=np.uint16) for n in lens]
    v_seq = [rng.integers(0, 2 ** 16, size=(n, 2, 64), dtype=np.uint16) for n in lens]
    for trial in range(3):
        perm = rng.permutation(12)
        tables = [list(perm[:3]), list(perm[3:6])]
        kp = np.zeros(spec.elements(), np.uint16)
        vp = np.zeros(spec.elements(), np.uint16)
        for b in range(2):
            for p in range(lens[b]):
                blk, t = divmod(slot(tables[b], p), 16)
                for h in range(2):
                    kp[k_element_offsets(spec, 1, blk, h, t)] = k_seq[b][p, h]
                    vp[v_element_offsets(spec, 1, blk, h, t)] = v_seq[b][p, h]
        for b in range(2):
            k, v = gather_sequence(kp, vp, spec, 1, tables[b], lens[b])
            assert np.array_equal(k, k_seq[b]) and np.array_equal(v, v_seq[b])


def test_interleaved_strides():
    # K and V interleaved per block in one array: k base 0, v base H*16*d.
    spec = PoolSpec(1, 4, 2, 64, "bf16", layer_stride=4 * 2 * 2 * 1024,
                    block_stride=2 * 2 * 1024, head_stride=1024)
    assert spec.plane_base(0, 3, 1) == 3 * 4096 + 1024
    assert spec.elements() == 3 * 4096 + 1024 + 1024


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 128), ("f16", 64)])
def test_plane_gather_equals_element_gather(dtype, d):
    from oracle.layout import gather_sequence_planes
    spec = PoolSpec(2, 9, 3, d, dtype, layer_stride=9 * 2 * 3 * 16 * d,
                    block_stride=2 * 3 * 16 * d, head_stride=16 * d)
    rng = np.random.default_rng(11)
    sdt = spec.storage_dtype()
    buf = (rng.integers(0, 2 ** 16, size=spec.elements() + 3 * 16 * d).astype(sdt)
           if sdt == np.uint16 else rng.standard_normal(spec.elements() + 3 * 16 * d).astype(sdt))
    kp, vp = buf, buf[3 * 16 * d:]
    row = [4, 0, 7, 2, -1]
    for n in (1, 16, 17, 50, 64):
        a = gather_sequence(kp, vp, spec, 1, row, n, heads=[2, 0])
        b = gather_sequence_planes(kp, vp, spec, 1, row, n, heads=[2, 0])
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
