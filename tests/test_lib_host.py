"""The C-ABI library on the CPU: it loads, exports every symbol the header
declares, and its host logic (allocator, rotary table, size formula, decode
split planner, argument checks) matches the oracle bit for bit.  No call
here touches a GPU."""

import ctypes
import os
import re

import numpy as np
import pytest

import paged_kv_cache_inject_amd as pkv
from oracle.allocator import AllocatorModel, AllocError, expand_table
from oracle.kv_size import kv_bytes
from oracle.rope import rope_rows, rope_table
from tests.conftest import ROOT


def header_functions():
    text = open(os.path.join(ROOT, "include", "pkv.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_[a-z0-9_]+)\s*\(", text)))


def test_library_loads_and_exports_every_declared_symbol():
    lib = pkv.load_library()
    names = header_functions()
    assert len(names) >= 20
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(pkv.SIGNATURES), set(names) ^ set(pkv.SIGNATURES)
    header = open(os.path.join(ROOT, "include", "pkv.h")).read()
    version = int(re.search(r"#define PKV_ABI_VERSION (\d+)", header).group(1))
    assert pkv.pkv_abi_version() == version


def test_kv_bytes_matches_closed_form():
    for args in [(80, 8, 128, 2, 8192), (32, 8, 128, 2, 1024), (12, 12, 64, 4, 1), (0, 1, 1, 1, 1)]:
        assert pkv.pkv_kv_bytes(*args) == kv_bytes(*args)
    assert pkv.pkv_kv_bytes(1, 1, 1, 1, -1) == 0


@pytest.mark.parametrize("d,max_pos", [(64, 128), (128, 4096), (128, 32768 + 64)])
def test_rope_table_bitwise_equal_to_oracle(d, max_pos):
    """Every row up to 4096, then every 13th row and the last 512 rows (the
    whole table at 32k positions costs minutes of float64 cos/sin on a slow
    host)."""
    c, s = pkv.pkv_rope_table(d, 10000.0, max_pos)
    rows = np.arange(max_pos)
    if max_pos > 4096:
        rows = np.unique(np.concatenate([rows[:4096], rows[4096::13], rows[-512:]]))
    oc, os_ = rope_rows(d, 10000.0, rows)
    assert np.array_equal(c[rows].view(np.uint32), oc.view(np.uint32))
    assert np.array_equal(s[rows].view(np.uint32), os_.view(np.uint32))


def test_worked_example_through_the_abi():
    c = pkv.pkv_cache_create(12, 2, 8)
    pkv.pkv_set_blocks(c, 0, [3, 7, 1], 40)
    pkv.pkv_set_blocks(c, 1, [2, 9], 20)
    assert pkv.pkv_free_list(c) == [0, 4, 5, 6, 8, 10, 11]
    first = pkv.pkv_extend(c, [1], 13)
    t, lens = pkv.pkv_block_table(c, [0, 1], 8)
    assert list(first) == [20] and list(lens) == [40, 33]
    assert list(t[1][:3]) == [2, 9, 0]
    pkv.pkv_cache_destroy(c)


def _unpad(row):
    """A table row without its trailing -1 padding (holes a window trim left
    at the front stay)."""
    row = [int(x) for x in row]
    while row and row[-1] < 0:
        row.pop()
    return row


def _state(c, model, max_b):
    """Library state next to the model's: exported plane tables (without
    padding), lengths, free list.  Returns the model's tables in the same
    plane form as the fourth item."""
    t, lens = pkv.pkv_block_table(c, list(range(model.max_seqs)), max_b * model.bt // 16)
    planes = [_unpad(expand_table(row, model.bt)) for row in model.tables]
    return ([_unpad(r) for r in t], list(lens), pkv.pkv_free_list(c), planes)


@pytest.mark.parametrize("seed", [0, 1, 12345])
def test_allocator_matches_oracle_on_random_operations(seed):
    rng = np.random.default_rng(seed + 7)
    nb, ns, mb = 40, 5, 12
    c = pkv.pkv_cache_create(nb, ns, mb, free_list_seed=seed)
    m = AllocatorModel(nb, ns, mb, seed=seed)
    assert pkv.pkv_free_list(c) == list(m.free)
    for step in range(400):
        op = rng.integers(0, 4)
        s = int(rng.integers(0, ns))
        err_c = err_m = None
        try:
            if op == 0:
                n = int(rng.integers(0, 120))
                try:
                    pkv.pkv_alloc_blocks(c, s, n)
                except pkv.PkvError as e:
                    err_c = e.code
                try:
                    m.alloc_blocks(s, n)
                except AllocError as e:
                    err_m = e.code
            elif op == 1:
                seqs = sorted(set(rng.integers(0, ns, size=int(rng.integers(1, 4))).tolist()))
                n = int(rng.integers(0, 40))
                try:
                    first = list(pkv.pkv_extend(c, seqs, n))
                except pkv.PkvError as e:
                    err_c, first = e.code, None
                try:
                    mfirst = m.extend(seqs, n)
                except AllocError as e:
                    err_m, mfirst = e.code, None
                assert first == mfirst
            elif op == 2:
                pkv.pkv_free_seq(c, s)
                m.free_seq(s)
            else:
                ids = list(m.free)[:int(rng.integers(0, 4))]
                ids = [int(x) for x in rng.permutation(ids)] if ids else []
                ln = int(rng.integers(0, 16 * len(ids) + 1))
                try:
                    pkv.pkv_set_blocks(c, s, ids, ln)
                except pkv.PkvError as e:
                    err_c = e.code
                try:
                    m.set_blocks(s, ids, ln)
                except AllocError as e:
                    err_m = e.code
        finally:
            pass
        assert err_c == err_m, (step, op, err_c, err_m)
        tables, lens, free, planes = _state(c, m, mb)
        assert tables == planes and lens == m.lens and free == list(m.free), step
        m.check_invariants()
    pkv.pkv_cache_destroy(c)


def _both(fc, fm):
    """Run the same operation on the library and on the model; return the
    two error codes (None when it succeeded) and the two results."""
    rc = rm = ec = em = None
    try:
        rc = fc()
    except pkv.PkvError as e:
        ec = e.code
    try:
        rm = fm()
    except AllocError as e:
        em = e.code
    return ec, em, rc, rm


@pytest.mark.parametrize("seed,bt", [(0, 16), (3, 16), (77, 16), (5, 32), (9, 32)])
def test_sharing_and_prefix_cache_match_oracle_on_random_operations(seed, bt):
    """Fork, copy-on-write on extend, free, prefix match and commit through
    the C ABI against the oracle model: tables, lengths, free list, reference
    counts, the copy queue and the cache size agree after every step (the
    queue is compared, never carried out, so nothing runs on a GPU)."""
    rng = np.random.default_rng(seed + 11)
    nb, ns, mb = 48, 6, 10
    c = pkv.pkv_cache_create(nb, ns, mb, free_list_seed=seed, block_tokens=bt)
    m = AllocatorModel(nb, ns, mb, seed=seed, block_tokens=bt)
    history = []                                   # key lists committed so far
    counts = dict(fork=0, cow=0, hit=0)
    for step in range(600):
        op = int(rng.integers(0, 8))
        s = int(rng.integers(0, ns))
        if op == 7:
            # capacity past the length, which a later fork shares
            n = m.lens[s] + int(rng.choice([1, 16, 40]))
            ec, em, _, _ = _both(lambda: pkv.pkv_alloc_blocks(c, s, n),
                                 lambda: m.alloc_blocks(s, n))
            counts["reserve"] = counts.get("reserve", 0) + (ec is None)
        elif op == 6:
            w = int(rng.choice([1, 10, 40]))
            ec, em, rc, rm = _both(lambda: pkv.pkv_trim_window(c, [s], w),
                                   lambda: m.trim_window([s], w))
            assert rc == rm
            counts["trim"] = counts.get("trim", 0) + (rc or 0)
        elif op == 0:
            seqs = sorted(set(rng.integers(0, ns, size=int(rng.integers(1, 3))).tolist()))
            n = int(rng.choice([1, 5, 16, 23]))
            ec, em, rc, rm = _both(lambda: list(pkv.pkv_extend(c, seqs, n)),
                                   lambda: m.extend(seqs, n))
            assert rc == rm
        elif op == 1:
            empty = [x for x in range(ns) if not m.tables[x] and x != s]
            d = int(rng.choice(empty)) if empty and rng.random() < 0.9 else int(rng.integers(0, ns))
            ec, em, _, _ = _both(lambda: pkv.pkv_fork(c, s, d), lambda: m.fork(s, d))
            counts["fork"] += ec is None
        elif op == 2:
            ec, em, _, _ = _both(lambda: pkv.pkv_free_seq(c, s), lambda: m.free_seq(s))
        elif op == 3:
            ln = m.lens[s]
            keys = [int(x) for x in rng.integers(0, 50, size=ln)] if ln else []
            if history and rng.random() < 0.7:
                base = history[int(rng.integers(0, len(history)))]
                keys = list(base[:ln]) + keys[len(base):]
            if len(keys) > ln:
                keys = keys[:ln]
            n_keys = int(rng.integers(0, ln + 1)) if ln else 0
            ec, em, _, _ = _both(lambda: pkv.pkv_prefix_commit(c, s, keys[:n_keys]),
                                 lambda: m.prefix_commit(s, keys[:n_keys]))
            if ec is None and n_keys >= bt:
                history.append(keys[:n_keys])
        else:
            if history and rng.random() < 0.8:
                keys = list(history[int(rng.integers(0, len(history)))])
                if rng.random() < 0.3 and keys:
                    keys[int(rng.integers(0, len(keys)))] ^= 1 << 40
            else:
                keys = [int(x) for x in rng.integers(0, 50, size=int(rng.integers(0, 60)))]
            keys = keys + [int(x) for x in rng.integers(0, 2 ** 63, size=int(rng.integers(0, 20)))]
            ec, em, rc, rm = _both(lambda: pkv.pkv_prefix_match(c, s, keys),
                                   lambda: m.prefix_match(s, keys))
            assert rc == rm
            counts["hit"] += bool(rc)
        assert ec == em, (step, op, ec, em)
        tables, lens, free, planes = _state(c, m, mb)
        assert tables == planes and lens == m.lens and free == list(m.free), step
        assert [pkv.pkv_block_refcount(c, b) for b in range(nb)] == m.ref, step
        assert pkv.pkv_pending_copies(c) == m.pending, step
        assert pkv.pkv_prefix_cached_blocks(c) == len(m.entries), step
        m.check_invariants()
    counts["cow"] = len(m.pending)
    assert counts["fork"] > 30 and counts["hit"] > (2 if bt == 16 else 1) and counts["cow"] > 8, counts
    assert counts.get("reserve", 0) > 30, counts
    assert counts.get("trim", 0) > 5, counts
    pkv.pkv_cache_destroy(c)


@pytest.mark.parametrize("length,n_new", [(32, 1), (30, 5), (48, 20)])
def test_extend_copies_reserved_shared_blocks_through_the_abi(length, n_new):
    """After a fork the sharers' reserved blocks past the length are shared
    too; extending both must leave each new position in a block of its own
    sequence (entries differ, count 1), as the oracle model says."""
    c = pkv.pkv_cache_create(16, 4, 8)
    m = AllocatorModel(16, 4, 8)
    for f in (lambda: pkv.pkv_set_blocks(c, 0, [3, 5, 7, 9], length),
              lambda: m.set_blocks(0, [3, 5, 7, 9], length)):
        f()
    pkv.pkv_fork(c, 0, 1)
    m.fork(0, 1)
    assert list(pkv.pkv_extend(c, [0, 1], n_new)) == m.extend([0, 1], n_new)
    table, _ = pkv.pkv_block_table(c, [0, 1])
    for i in range(length // 16, -(-(length + n_new) // 16)):
        a, b = int(table[0][i]), int(table[1][i])
        assert a != b and pkv.pkv_block_refcount(c, a) == 1 and pkv.pkv_block_refcount(c, b) == 1
    assert pkv.pkv_pending_copies(c) == m.pending
    assert _unpad(table[0]) == m.tables[0] and _unpad(table[1]) == m.tables[1]
    pkv.pkv_cache_destroy(c)


def test_window_trim_through_the_abi():
    c = pkv.pkv_cache_create(32, 2, 16)
    m = AllocatorModel(32, 2, 16)
    pkv.pkv_extend(c, [0], 100)
    m.extend([0], 100)
    assert pkv.pkv_trim_window(c, [0], 20) == m.trim_window([0], 20) == 5
    t, lens = pkv.pkv_block_table(c, [0], 16)
    assert list(t[0][:5]) == [-1] * 5 and list(t[0]) == m.tables[0] + [-1] * (16 - 7)
    assert pkv.pkv_free_list(c) == list(m.free)
    for bad in (0, -3):
        with pytest.raises(pkv.PkvError) as e:
            pkv.pkv_trim_window(c, [0], bad)
        assert e.value.code == "INVALID"
    with pytest.raises(pkv.PkvError) as e:
        pkv.pkv_prefix_commit(c, 0, list(range(32)))   # keys over dropped blocks
    assert e.value.code == "RANGE"
    pkv.pkv_free_seq(c, 0)
    assert pkv.pkv_num_free_blocks(c) == 32
    pkv.pkv_cache_destroy(c)


def test_sharing_errors_through_the_abi():
    c = pkv.pkv_cache_create(4, 3, 4)
    pkv.pkv_extend(c, [0], 40)
    for args in [(0, 0), (0, 7), (-1, 1)]:
        with pytest.raises(pkv.PkvError) as e:
            pkv.pkv_fork(c, *args)
        assert e.value.code == "INVALID"
    pkv.pkv_fork(c, 0, 1)
    with pytest.raises(pkv.PkvError) as e:
        pkv.pkv_prefix_match(c, 1, list(range(16)))    # not empty
    assert e.value.code == "INVALID"
    with pytest.raises(pkv.PkvError) as e:
        pkv.pkv_prefix_commit(c, 0, list(range(41)))   # more keys than tokens
    assert e.value.code == "RANGE"
    pkv.pkv_fork(c, 0, 2)
    with pytest.raises(pkv.PkvError) as e:
        pkv.pkv_extend(c, [1, 2], 1)                   # two copies, one free block
    assert e.value.code == "OOM"
    assert pkv.pkv_pending_copies(c) == [] and pkv.pkv_num_free_blocks(c) == 1
    with pytest.raises(pkv.PkvError) as e:
        pkv.pkv_block_refcount(c, 4)
    assert e.value.code == "INVALID"
    pkv.pkv_cache_destroy(c)


def test_seeded_free_list_matches_oracle_at_workload_size():
    from workloads.configs import inject_structure
    st = inject_structure(n_chunks=50)
    c = pkv.pkv_cache_create(st["num_blocks"], 64, st["max_blocks"], st["free_list_seed"])
    m = AllocatorModel(st["num_blocks"], 64, st["max_blocks"], seed=st["free_list_seed"])
    assert pkv.pkv_free_list(c) == list(m.free)
    for b, ml in enumerate(st["mem_lens"]):
        pkv.pkv_alloc_blocks(c, b, int(ml))
        m.alloc_blocks(b, int(ml))
    tables, _, free, planes = _state(c, m, st["max_blocks"])
    assert tables == planes and free == list(m.free)


def test_decode_plan_splits():
    lens = [37, 100, 0, 5000, 16, 17]
    plan = pkv.pkv_decode_plan_create(lens, 4, 2, 64, 32)
    # ceil(len / 32) ranges per sequence; an empty sequence is one empty item
    assert pkv.pkv_decode_plan_items(plan) == sum(max(1, -(-x // 32)) for x in lens)
    assert pkv.pkv_decode_plan_waves(plan) in (1, 2, 4, 8)
    assert pkv.pkv_decode_plan_part_tokens(plan) == 32
    assert pkv.pkv_decode_workspace_bytes(plan) % 256 == 0
    pkv.pkv_decode_plan_destroy(plan)
    plan = pkv.pkv_decode_plan_create([8192] * 32, 64, 8, 128, 0)
    # 32 x 8 (sequence, KV head) pairs of 512 blocks: one 8-wave workgroup each
    assert pkv.pkv_decode_plan_waves(plan) == 8
    assert pkv.pkv_decode_plan_items(plan) == 32
    pkv.pkv_decode_plan_destroy(plan)
    for bad in [dict(part=8), dict(hq=6, hkv=4), dict(d=96)]:
        with pytest.raises(pkv.PkvError):
            pkv.pkv_decode_plan_create([10], bad.get("hq", 4), bad.get("hkv", 2),
                                       bad.get("d", 64), bad.get("part", 0))


def test_small_plan_upload_enqueues_nothing():
    """A plan of at most 128 items that splits no sequence travels in the
    decode launch's kernel arguments: its upload only validates the
    workspace (a fake, aligned device address is never touched)."""
    fake = 1 << 20
    plan = pkv.pkv_decode_plan_create([40] * 128, 8, 2, 64, 0)
    try:
        assert pkv.pkv_decode_plan_items(plan) == 128
        n = pkv.pkv_decode_workspace_bytes(plan)
        lib = pkv.load_library()
        assert lib.pkv_decode_plan_upload(plan, fake, n, None) == 0
        # the workspace is still checked
        assert lib.pkv_decode_plan_upload(plan, fake, n - 1, None) < 0
        assert lib.pkv_decode_plan_upload(plan, fake + 16, n, None) < 0
    finally:
        pkv.pkv_decode_plan_destroy(plan)


def test_append_decode_host_validation_errors():
    """The one-launch append and decode checks its new-token arguments on
    the host before any device work (fake device pointers, never read)."""
    import torch
    fake = 1 << 20
    pool = pkv.pkv_pool(1, 8, 2, 64, pkv.PKV_BF16, 0, fake, fake + 4096, 8 * 4096, 4096, 1024)
    plan = pkv.pkv_decode_plan_create([10, 60], 4, 2, 64, 0)
    tables = np.zeros((2, 8), dtype=np.int32)
    ws = torch.empty(pkv.pkv_decode_workspace_bytes(plan), dtype=torch.uint8)

    def call(k_new=fake, v_new=fake, mode="pairs", max_pos=100, q_dtype="bf16"):
        pkv.pkv_append_decode_attention(plan, pool, 0, fake, tables, k_new, v_new, mode, fake, fake,
                                        max_pos, fake, fake, ws, stream=0, q_dtype=q_dtype)

    cases = [(dict(k_new=None), "INVALID"), (dict(v_new=None), "INVALID"),
             (dict(k_new=fake + 2), "INVALID"), (dict(mode=7), "INVALID"),
             (dict(max_pos=59), "RANGE"), (dict(max_pos=-1), "INVALID"),
             (dict(q_dtype="f16"), "UNSUPPORTED")]
    for kw, code in cases:
        with pytest.raises(pkv.PkvError) as e:
            call(**kw)
        assert e.value.code == code, (kw, e.value.code)
    pkv.pkv_decode_plan_destroy(plan)


def test_empty_batch_calls_need_no_device_arguments():
    """Calls with nothing to do return success on the host and enqueue
    nothing, whatever their device pointers: decode and the fused step over a
    plan of no sequences, an append for no sequences or of no tokens, an
    inject call with no runs or only empty runs (null device pointers, never
    dereferenced; no device is needed)."""
    import ctypes
    lib = pkv.load_library()
    fake = 1 << 20
    pool = pkv.pkv_pool(1, 8, 2, 64, pkv.PKV_BF16, 0, fake, fake + 4096, 8 * 4096, 4096, 1024)
    none = pkv.ROPE_CODES["none"]
    plan = pkv.pkv_decode_plan_create(np.zeros(0, np.int64), 4, 2, 64, 0)
    try:
        assert lib.pkv_decode_attention(plan, ctypes.byref(pool), 0, None, pkv.PKV_BF16, 0.0,
                                        None, 8, None, None, None, 0, None) == 0
        assert lib.pkv_append_decode_attention(plan, ctypes.byref(pool), 0, None, pkv.PKV_BF16,
                                               0.0, None, 8, None, None, none, None, None, 0,
                                               None, None, None, 0, None) == 0
    finally:
        pkv.pkv_decode_plan_destroy(plan)
    for n_seqs, n_new in ((0, 1), (3, 0)):
        assert lib.pkv_append_kv(ctypes.byref(pool), 0, None, 8, None, n_seqs, n_new, None, None,
                                 pkv.PKV_BF16, none, None, None, 0, None) == 0
    src = pkv.pkv_src(fake, fake, 0, 128, 64, pkv.PKV_BF16)
    c = pkv.pkv_cache_create(8, 2, 4)
    try:
        pkv.pkv_alloc_blocks(c, 0, 20)
        for runs in ([], [(0, 0, 0, 0), (0, 0, 500, 0), (1, 0, 7, 9)]):
            arr = pkv.make_runs(runs) if runs else None
            assert lib.pkv_inject(c, ctypes.byref(pool), ctypes.byref(src), arr, len(runs), 0, 1,
                                  none, None, None, 0, None, 0, None) == 0, pkv.pkv_last_error()
        _, lens = pkv.pkv_block_table(c, range(2))
        assert list(lens) == [0, 0]
    finally:
        pkv.pkv_cache_destroy(c)


def test_inject_host_validation_errors():
    """Argument errors are found on the host before any device work (the
    fake device pointers below are never dereferenced)."""
    fake = 1 << 20
    pool = pkv.pkv_pool(1, 8, 2, 64, pkv.PKV_BF16, 0, fake, fake + 4096, 8 * 4096, 4096, 1024)
    src = pkv.pkv_src(fake, fake, 0, 128, 64, pkv.PKV_BF16)
    c = pkv.pkv_cache_create(8, 2, 4)
    pkv.pkv_alloc_blocks(c, 0, 40)
    cases = [([(0, 4, 0, 0), (0, 4, 2, 10)], "OVERLAP"), ([(0, 10, 40, 0)], "RANGE"),
             ([(0, 10, 0, 60)], "RANGE"), ([(1, 1, 0, 0)], "RANGE"), ([(5, 1, 0, 0)], "INVALID"),
             ([(0, -1, 0, 0)], "INVALID")]
    for runs, code in cases:
        with pytest.raises(pkv.PkvError) as e:
            pkv.pkv_inject(c, pool, src, runs, 0, 1, "pairs", fake, fake, 100, None, stream=0)
        assert e.value.code == code
    bad_pool = pkv.pkv_pool(1, 8, 2, 96, pkv.PKV_BF16, 0, fake, fake, 0, 0, 0)
    with pytest.raises(pkv.PkvError) as e:
        pkv.pkv_inject(c, bad_pool, src, [(0, 1, 0, 0)], 0, 1, "pairs", fake, fake, 100, None,
                       stream=0)
    assert e.value.code == "UNSUPPORTED"
    no_scales = pkv.pkv_pool(1, 8, 2, 64, pkv.PKV_FP8E4M3, 0, fake, fake, 0, 2048, 1024)
    with pytest.raises(pkv.PkvError) as e:       # an fp8 pool needs its scales
        pkv.pkv_inject(c, no_scales, src, [(0, 1, 0, 0)], 0, 1, "pairs", fake, fake, 100, None,
                       stream=0)
    assert e.value.code == "INVALID"
    # a source in pageable host memory is refused before anything is enqueued
    import torch
    host = np.zeros(64 * 128, dtype=np.uint16)
    pageable = pkv.pkv_src(host.ctypes.data, host.ctypes.data, 0, 128, 64, pkv.PKV_BF16)
    ws = torch.empty(pkv.pkv_inject_workspace_bytes([(0, 4, 0, 0)]), dtype=torch.uint8)
    with pytest.raises(pkv.PkvError) as e:
        pkv.pkv_inject(c, pool, pageable, [(0, 4, 0, 0)], 0, 1, "pairs", fake, fake, 100, ws,
                       stream=0)
    assert e.value.code == "INVALID" and "pinned" in str(e.value)
    _, lens = pkv.pkv_block_table(c, [0], 4)
    assert list(lens) == [0]
    fp8_pool = pkv.pkv_pool(1, 8, 2, 64, pkv.PKV_FP8E4M3, 0, fake, fake, 0, 2048, 1024, fake, fake)
    f32_src = pkv.pkv_src(fake, fake, 0, 128, 64, pkv.PKV_F32)
    with pytest.raises(pkv.PkvError) as e:       # f32 sources are not quantised
        pkv.pkv_inject(c, fp8_pool, f32_src, [(0, 1, 0, 0)], 0, 1, "pairs", fake, fake, 100,
                       None, stream=0)
    assert e.value.code == "UNSUPPORTED"
    f16_src = pkv.pkv_src(fake, fake, 0, 128, 64, pkv.PKV_F16)
    with pytest.raises(pkv.PkvError) as e:       # a bf16 pool takes bf16 sources only
        pkv.pkv_inject(c, pool, f16_src, [(0, 1, 0, 0)], 0, 1, "pairs", fake, fake, 100, None,
                       stream=0)
    assert e.value.code == "UNSUPPORTED"
    misaligned = pkv.pkv_pool(1, 8, 2, 64, pkv.PKV_BF16, 0, fake + 2, fake, 0, 4096, 1024)
    with pytest.raises(pkv.PkvError) as e:
        pkv.pkv_inject(c, misaligned, src, [(0, 1, 0, 0)], 0, 1, "pairs", fake, fake, 100, None,
                       stream=0)
    assert e.value.code == "INVALID"
    with pytest.raises(pkv.PkvError) as e:      # needs a workspace
        pkv.pkv_inject(c, pool, src, [(0, 1, 0, 0)], 0, 1, "pairs", fake, fake, 100, None,
                       stream=0)
    assert e.value.code == "WORKSPACE"
    _, lens = pkv.pkv_block_table(c, [0], 4)
    assert list(lens) == [0]
    pkv.pkv_cache_destroy(c)


def test_cache_facade_is_the_handle_calls():
    with pkv.Cache(16, 3, 8, free_list_seed=3) as c:
        m = AllocatorModel(16, 3, 8, seed=3)
        assert c.extend([0], 40).tolist() == m.extend([0], 40)
        c.fork(0, 1)
        m.fork(0, 1)
        c.extend([1], 1)
        m.extend([1], 1)
        assert c.pending_copies() == m.pending
        assert c.free_list() == list(m.free) and c.num_free_blocks() == len(m.free)
        t, lens = c.block_table([0, 1])
        assert [_unpad(r) for r in t] == m.tables[:2] and list(lens) == m.lens[:2]
        c.prefix_commit(0, list(range(32)))
        m.prefix_commit(0, list(range(32)))
        assert c.prefix_cached_blocks() == len(m.entries) == 2
        assert c.trim_window([0], 10) == m.trim_window([0], 10)
        assert [c.block_refcount(b) for b in range(16)] == m.ref
        assert c.table_width() == 8
    assert c.handle is None


def test_kernel_timing_helper_without_launches():
    """The timing helper returns nothing recorded when nothing was launched,
    and rejects a missing output buffer."""
    assert len(pkv.pkv_kernel_times()) == 0
    pkv.pkv_kernel_timing(True)
    pkv.pkv_kernel_timing(False)
    assert len(pkv.pkv_kernel_times()) == 0
    assert pkv.load_library().pkv_kernel_times(None, 4) == pkv.PKV_E_INVALID


def test_inject_overlap_found_in_any_plane_and_scale_mode_checked():
    """The planner walks each run a 16-token plane at a time: a second write
    to a slot is found wherever it falls (first plane, a later plane, the
    second plane of a 32-token block); a pool's scale_mode is 0, or 1 for an
    fp8 pool only."""
    fake = 1 << 20
    pool = pkv.pkv_pool(1, 16, 2, 64, pkv.PKV_BF16, 0, fake, fake + 4096, 16 * 4096, 4096, 1024)
    src = pkv.pkv_src(fake, fake, 0, 128, 256, pkv.PKV_BF16)
    for bt in (16, 32):
        c = pkv.pkv_cache_create(8, 2, 8, block_tokens=bt)   # 8 blocks = up to 16 planes
        pkv.pkv_alloc_blocks(c, 0, 100)
        for runs in ([(0, 10, 12, 0), (0, 3, 18, 50)],      # second plane of the first run
                     [(0, 40, 3, 0), (0, 1, 42, 90)],       # third plane
                     [(0, 20, 20, 0), (0, 2, 38, 90)],      # 32-token block, its second plane
                     [(0, 5, 0, 0), (0, 1, 4, 90)]):        # first plane
            with pytest.raises(pkv.PkvError) as e:
                pkv.pkv_inject(c, pool, src, runs, 0, 1, "pairs", fake, fake, 200, None, stream=0)
            assert e.value.code == "OVERLAP", (bt, runs)
        # nothing was planned or kept: the sequence is still empty
        _, lens = pkv.pkv_block_table(c, [0], pkv.pkv_table_width(c))
        assert list(lens) == [0]
        pkv.pkv_cache_destroy(c)
    c = pkv.pkv_cache_create(8, 2, 4)
    pkv.pkv_alloc_blocks(c, 0, 40)
    for dtype, mode, scales in ((pkv.PKV_BF16, 1, None), (pkv.PKV_FP8E4M3, 2, fake),
                                (pkv.PKV_BF16, -1, None)):
        bad = pkv.pkv_pool(1, 8, 2, 64, dtype, mode, fake, fake + 4096, 8 * 4096, 4096, 1024,
                           scales, scales)
        with pytest.raises(pkv.PkvError) as e:
            pkv.pkv_inject(c, bad, src, [(0, 1, 0, 0)], 0, 1, "pairs", fake, fake, 100, None,
                           stream=0)
        assert e.value.code == "INVALID" and "scale_mode" in str(e.value)
    pkv.pkv_cache_destroy(c)
