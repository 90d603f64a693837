"""Write side on the GPU against the oracle, byte for byte: inject (aligned
and unaligned runs, partial blocks, overwrites, every dtype and rotary
mode) and append (T = 1, 17, 32, crossing block boundaries)."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

CANARY = {"f32": 0x7FC0DEAD, "bf16": 0x7FAB, "f16": 0x7DAB, "fp8": 0x5A}


def canary_buffer(dp, dtype):
    if dtype == "f32":
        return np.full(dp.total, np.uint32(CANARY[dtype]).view(np.float32), dtype=np.float32)
    if dtype == "fp8":
        return np.full(dp.total, CANARY[dtype], dtype=np.uint8)
    return np.full(dp.total, CANARY[dtype], dtype=np.uint16)


@pytest.mark.parametrize("dtype,d,mode", [
    ("bf16", 128, "pairs"), ("bf16", 128, "halves"), ("bf16", 128, "none"),
    ("f16", 128, "pairs"), ("f16", 64, "halves"), ("bf16", 64, "pairs"),
    ("f32", 128, "pairs"), ("f32", 64, "halves"),
])
def test_inject_matches_oracle(dtype, d, mode):
    import torch
    import paged_kv_cache_inject_amd as pkv
    from oracle import inject as o_inject
    from oracle.allocator import AllocatorModel
    from oracle.rope import rope_table
    from tests import gpu_util as gu
    from workloads.configs import host_normal

    gu.say("inject", dtype, d, mode)
    rng = np.random.default_rng(hash((dtype, d, mode)) % 2 ** 32)
    L, H, NB, max_pos = 3, 4, 48, 300
    dp = gu.DevicePool(L, NB, H, d, dtype, fill_bits=CANARY[dtype])
    cache = pkv.pkv_cache_create(NB, 4, 16, free_list_seed=77)
    model = AllocatorModel(NB, 4, 16, seed=77)
    for s, n in enumerate((100, 37, 250, 16)):
        pkv.pkv_alloc_blocks(cache, s, n)
        model.alloc_blocks(s, n)
    t, _ = pkv.pkv_block_table(cache, range(4), 16)
    assert [list(r[r >= 0]) for r in t] == model.tables
    n_src = 400
    src_k = host_normal(rng, (L, n_src, H, d), dtype)
    src_v = host_normal(rng, (L, n_src, H, d), dtype)
    calls = [
        [(0, 100, 0, 0), (1, 37, 0, 100), (3, 16, 0, 137)],                 # aligned prefill
        [(2, 5, 3, 200), (2, 40, 9, 153), (2, 1, 250 - 1, 399),             # unaligned, partial
         (2, 100, 60, 210), (0, 24, 40, 300), (1, 2, 35, 330)],              # overwrites
        [(2, 0, 0, 0), (1, 1, 0, 398)],                                      # empty run, one token
        [(0, 64, 0, 5)],       # 4 destination blocks: descriptors in the kernel arguments
        [(0, 65, 0, 6)],       # 5 destination blocks: descriptors through the workspace
    ]
    o_cos, o_sin = rope_table(d, 10000.0, max_pos)
    cos, sin, dcos, dsin = gu.rope_tables(d, max_pos)
    assert np.array_equal(cos, o_cos) and np.array_equal(sin, o_sin)
    dk = gu.to_device_raw(src_k.reshape(-1), dtype)
    dv = gu.to_device_raw(src_v.reshape(-1), dtype)
    src = pkv.make_src(dk, dv, n_src * H * d, H * d, n_src)
    ref = canary_buffer(dp, dtype)
    kp, vp = dp.oracle_arrays(ref)
    lens = [0] * 4
    for i, runs in enumerate(calls):
        lb, le = (0, L) if i != 1 else (1, L)        # one call on a layer range
        ws = gu.workspace(pkv.pkv_inject_workspace_bytes(runs))
        pkv.pkv_inject(cache, dp.desc(), src, runs, lb, le, mode, dcos, dsin, max_pos, ws)
        torch.cuda.synchronize()
        lens = o_inject.inject(kp, vp, dp.spec(), model.tables, lens, runs, src_k.reshape(-1),
                               src_v.reshape(-1), n_src * H * d, H * d, lb, le, mode, o_cos, o_sin)
        gu.assert_bytes_equal(dp.host_copy(), ref, "pool after inject call %d" % i)
    _, glens = pkv.pkv_block_table(cache, range(4), 16)
    assert list(glens) == lens


def test_inject_rejects_overlap_and_range_without_enqueueing():
    import torch
    import paged_kv_cache_inject_amd as pkv
    from tests import gpu_util as gu

    dp = gu.DevicePool(1, 8, 2, 64, "bf16", fill_bits=0x1234)
    cache = pkv.pkv_cache_create(8, 2, 4)
    pkv.pkv_alloc_blocks(cache, 0, 40)
    src_t = torch.zeros(64 * 2 * 64, dtype=torch.bfloat16, device="cuda")
    src = pkv.make_src(src_t, src_t, 0, 128, 64)
    cos, sin, dcos, dsin = gu.rope_tables(64, 100)
    ws = gu.workspace(1 << 16)
    before = dp.host_copy()
    for runs, code in [([(0, 4, 0, 0), (0, 4, 2, 10)], "OVERLAP"),
                       ([(0, 10, 40, 0)], "RANGE"),
                       ([(0, 10, 95, 0)], "RANGE"),
                       ([(0, 10, 0, 60)], "RANGE"),
                       ([(1, 1, 0, 0)], "RANGE"),
                       ([(5, 1, 0, 0)], "INVALID")]:
        with pytest.raises(pkv.PkvError) as e:
            pkv.pkv_inject(cache, dp.desc(), src, runs, 0, 1, "pairs", dcos, dsin, 100, ws)
        assert e.value.code == code, (runs, e.value)
    torch.cuda.synchronize()
    gu.assert_bytes_equal(dp.host_copy(), before, "pool after rejected calls")
    _, lens = pkv.pkv_block_table(cache, [0, 1], 4)
    assert list(lens) == [0, 0]


@pytest.mark.parametrize("dtype,d,mode,n_new", [
    ("bf16", 128, "pairs", 1), ("bf16", 128, "pairs", 32), ("bf16", 128, "halves", 17),
    ("bf16", 128, "none", 1), ("f16", 128, "pairs", 32), ("f32", 64, "pairs", 3),
])
def test_append_matches_oracle(dtype, d, mode, n_new):
    import torch
    import paged_kv_cache_inject_amd as pkv
    from oracle import inject as o_inject
    from oracle.allocator import AllocatorModel
    from oracle.rope import rope_table
    from tests import gpu_util as gu
    from workloads.configs import host_normal

    gu.say("append", dtype, d, mode, n_new)
    rng = np.random.default_rng(n_new * 7 + d)
    L, H, NB, B, max_pos = 2, 8, 64, 6, 512
    dp = gu.DevicePool(L, NB, H, d, dtype, fill_bits=CANARY[dtype])
    cache = pkv.pkv_cache_create(NB, B, 32, free_list_seed=5)
    model = AllocatorModel(NB, B, 32, seed=5)
    start = [0, 15, 16, 31, 100, 47]
    for s, n in enumerate(start):
        pkv.pkv_extend(cache, [s], n)
        model.extend([s], n)
    seqs = list(range(B))
    first = pkv.pkv_extend(cache, seqs, n_new)
    assert list(first) == model.extend(seqs, n_new)
    table, lens = pkv.pkv_block_table(cache, seqs, 32)
    assert [list(r[r >= 0]) for r in table] == model.tables and list(lens) == model.lens
    o_cos, o_sin = rope_table(d, 10000.0, max_pos)
    _, _, dcos, dsin = gu.rope_tables(d, max_pos)
    ref = canary_buffer(dp, dtype)
    kp, vp = dp.oracle_arrays(ref)
    tables_dev = torch.from_numpy(table).cuda()
    first_dev = torch.from_numpy(first.astype(np.int32)).cuda()
    for layer in range(L):
        k_new = host_normal(rng, (B, n_new, H, d), dtype)
        v_new = host_normal(rng, (B, n_new, H, d), dtype)
        pkv.pkv_append_kv(dp.desc(), layer, tables_dev, first_dev, n_new,
                          gu.to_device_raw(k_new.reshape(-1), dtype),
                          gu.to_device_raw(v_new.reshape(-1), dtype), mode, dcos, dsin, max_pos)
        o_inject.append(kp, vp, dp.spec(), layer, model.tables, model.lens, seqs, n_new,
                        k_new, v_new, mode, o_cos, o_sin)
    torch.cuda.synchronize()
    gu.assert_bytes_equal(dp.host_copy(), ref, "pool after append")


@pytest.mark.parametrize("dtype,mode", [("bf16", "pairs"), ("bf16", "none"), ("f16", "halves"),
                                        ("fp8", "pairs")])
def test_append_skips_positions_the_device_data_does_not_cover(dtype, mode):
    """First positions and tables on the device are range-checked: tokens at
    negative positions, past the table row, past the rotary table (under a
    rotary pairing) or in a block whose id is out of range are not written;
    the other tokens of the same call are.  Pool byte-exact against the
    oracle's append over the same device data."""
    import torch
    import paged_kv_cache_inject_amd as pkv
    from oracle import inject as o_inject
    from oracle.rope import rope_table
    from tests import gpu_util as gu
    from workloads.configs import host_normal

    gu.say("append, out-of-range device data", dtype, mode)
    rng = np.random.default_rng(404)
    L, H, d, NB, W, max_pos, n_new = 2, 4, 128, 40, 4, 50, 8
    dp = gu.DevicePool(L, NB, H, d, dtype, fill_bits=CANARY[dtype])
    ks = vs = None
    if dtype == "fp8":
        ks = rng.uniform(0.01, 0.03, size=(L, H)).astype(np.float32)
        vs = rng.uniform(0.01, 0.03, size=(L, H)).astype(np.float32)
        dp.set_scales(ks, vs)
    # each row: W = 4 blocks of 16 positions (64 positions), distinct blocks
    ids = rng.permutation(NB)[:7 * W].astype(np.int32).reshape(7, W)
    table = ids.copy()
    table[5, 1] = NB + 3            # positions 16..31 of row 5 name no block
    table[6, 0] = -1
    # first positions: straddling 0; straddling max_pos; straddling the end of
    # the row; far past it; straddling a bad entry; inside; inside a bad entry
    first = np.array([-3, 46, 60, 2 ** 30, 12, 30, 4], dtype=np.int32)
    src_dt = "bf16" if dtype == "fp8" else dtype
    o_cos, o_sin = rope_table(d, 10000.0, max_pos)
    _, _, dcos, dsin = gu.rope_tables(d, max_pos)
    ref = canary_buffer(dp, dtype)
    kp, vp = dp.oracle_arrays(ref)
    tdev = torch.from_numpy(table).cuda()
    fdev = torch.from_numpy(first).cuda()
    rows = [list(r) for r in table]
    lens_after = [int(f) + n_new for f in first]
    for layer in range(L):
        k_new = host_normal(rng, (7, n_new, H, d), src_dt)
        v_new = host_normal(rng, (7, n_new, H, d), src_dt)
        pkv.pkv_append_kv(dp.desc(), layer, tdev, fdev, n_new,
                          gu.to_device_raw(k_new.reshape(-1), src_dt),
                          gu.to_device_raw(v_new.reshape(-1), src_dt), mode, dcos, dsin, max_pos,
                          new_dtype=src_dt)
        o_inject.append(kp, vp, dp.spec(), layer, rows, lens_after, list(range(7)), n_new, k_new,
                        v_new, mode, o_cos, o_sin, src_dtype=src_dt, k_scale=ks, v_scale=vs,
                        num_blocks=NB)
    torch.cuda.synchronize()
    got = dp.host_copy()
    gu.assert_bytes_equal(got, ref, "pool after append with out-of-range device data")
    # something was written, and the canary survives where nothing may be
    assert (got != canary_buffer(dp, dtype)).any()


@pytest.mark.parametrize("pf", ["0", "1"])
@pytest.mark.parametrize("dtype,src_dtype,d,mode", [
    ("bf16", "bf16", 128, "pairs"), ("fp8", "bf16", 128, "halves"), ("f32", "f32", 64, "none"),
    ("f16", "f16", 64, "pairs"),
])
def test_inject_layer_groups_with_and_without_prefetch(pf, dtype, src_dtype, d, mode):
    """Workgroups that walk several layers and heads: 8 KV heads (two per
    wave) and 5 layers per workgroup give each wave 10 (layer, head) steps,
    so the one-deep prefetch alternates its buffers and ends on an odd step;
    the same call without prefetch gives the same bytes.  Pool byte-exact
    against the oracle."""
    import os
    import torch
    import paged_kv_cache_inject_amd as pkv
    from oracle import inject as o_inject
    from oracle.allocator import AllocatorModel
    from oracle.rope import rope_table
    from tests import gpu_util as gu
    from workloads.configs import host_normal

    gu.say("inject layer groups", pf, dtype, src_dtype, d, mode)
    rng = np.random.default_rng(len(dtype) * 31 + d + len(mode) + int(pf))
    L, H, NB, max_pos = 5, 8, 40, 400
    dp = gu.DevicePool(L, NB, H, d, dtype, fill_bits=CANARY[dtype])
    ks = vs = None
    if dtype == "fp8":
        ks = rng.uniform(0.005, 0.03, size=(L, H)).astype(np.float32)
        vs = rng.uniform(0.005, 0.03, size=(L, H)).astype(np.float32)
        dp.set_scales(ks, vs)
    cache = pkv.pkv_cache_create(NB, 3, 16, free_list_seed=5)
    model = AllocatorModel(NB, 3, 16, seed=5)
    for s, n in enumerate((130, 61, 200)):
        pkv.pkv_alloc_blocks(cache, s, n)
        model.alloc_blocks(s, n)
    n_src = 500
    src_k = host_normal(rng, (L, n_src, H, d), src_dtype)
    src_v = host_normal(rng, (L, n_src, H, d), src_dtype)
    runs = [(0, 130, 0, 0), (1, 61, 0, 130), (2, 7, 0, 300), (2, 150, 7, 191), (2, 43, 157, 400)]
    o_cos, o_sin = rope_table(d, 10000.0, max_pos)
    _, _, dcos, dsin = gu.rope_tables(d, max_pos)
    dk = gu.to_device_raw(src_k.reshape(-1), src_dtype)
    dv = gu.to_device_raw(src_v.reshape(-1), src_dtype)
    src = pkv.make_src(dk, dv, n_src * H * d, H * d, n_src, dtype=src_dtype)
    ws = gu.workspace(pkv.pkv_inject_workspace_bytes(runs))
    os.environ["PKV_INJECT_LAYERS_PER_WG"] = "5"
    os.environ["PKV_INJECT_PREFETCH"] = pf
    try:
        pkv.pkv_inject(cache, dp.desc(), src, runs, 0, L, mode, dcos, dsin, max_pos, ws)
        torch.cuda.synchronize()
    finally:
        os.environ.pop("PKV_INJECT_LAYERS_PER_WG", None)
        os.environ.pop("PKV_INJECT_PREFETCH", None)
    ref = canary_buffer(dp, dtype)
    kp, vp = dp.oracle_arrays(ref)
    o_inject.inject(kp, vp, dp.spec(), model.tables, [0, 0, 0], runs, src_k.reshape(-1),
                    src_v.reshape(-1), n_src * H * d, H * d, 0, L, mode, o_cos, o_sin,
                    src_dtype=src_dtype, k_scale=ks, v_scale=vs)
    gu.assert_bytes_equal(dp.host_copy(), ref, "pool after a layer-group inject")
