"""Sliding-window decode on the GPU against the oracle ([KV essay] "Capping
the window instead of shrinking the rows"): every sequence attends to its
last W positions.  Edge lengths and windows (inside one block, on block
edges, longer than the sequence) at several split sizes, MFMA and VALU
kernels and an fp8 pool; a sequence grown token by token with its table
trimmed after every step, the dropped blocks reused by another sequence
that fills them with NaN; and writes into dropped positions refused."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

LENS = [0, 1, 15, 16, 17, 40, 100, 333, 700, 2000]


@pytest.mark.parametrize("dtype,hq,hkv,d", [("bf16", 32, 4, 128), ("f16", 8, 8, 64),
                                            ("f32", 4, 2, 64), ("fp8", 16, 2, 128),
                                            ("fp8b", 16, 2, 128)])
def test_window_decode_matches_oracle(dtype, hq, hkv, d):
    """("fp8b": an fp8 pool with scales per (layer, block, KV head).)"""
    import torch
    from oracle import attention as o_att
    from tests import gpu_util as gu
    from workloads.configs import host_normal, deal_tables

    gu.say("window decode", dtype, hq, hkv, d)
    rng = np.random.default_rng(hq * 3 + d + (dtype == "fp8b"))
    blockwise = dtype == "fp8b"
    dtype = "fp8" if blockwise else dtype
    lens = np.array(LENS, dtype=np.int64)
    need = int(sum(-(-x // 16) for x in lens))
    nb = need + 4
    table = deal_tables(rng.permutation(nb)[:need].astype(np.int32), lens, 128)
    dp = gu.DevicePool(1, nb, hkv, d, dtype)
    ks = vs = None
    if dtype == "fp8":
        shape = (1, nb, hkv) if blockwise else (1, hkv)
        ks = rng.uniform(0.01, 0.03, size=shape).astype(np.float32)
        vs = rng.uniform(0.01, 0.03, size=shape).astype(np.float32)
        dp.set_scales(ks, vs)
        codes = rng.integers(0, 0x60, size=dp.total, dtype=np.uint8)
        codes |= (rng.integers(0, 2, size=dp.total, dtype=np.uint8) << 7).astype(np.uint8)
        raw = codes
    else:
        raw = host_normal(rng, (dp.total,), dtype)
    dp.buf.copy_(gu.to_device_raw(raw, dtype))
    kp, vp = dp.oracle_arrays(raw)
    qdt = "bf16" if dtype == "fp8" else dtype
    q = host_normal(rng, (len(lens), hq, d), qdt)
    q_dev = gu.to_device_raw(q.reshape(-1), qdt).view(q.shape)
    tdev = torch.from_numpy(table).cuda()
    for w in (1, 7, 16, 17, 64, 500, 4096):
        ref, ref_lse = o_att.decode_paged(q, kp, vp, dp.spec(), 0, [list(r) for r in table], lens,
                                          hq, by_plane=True, q_dtype=qdt, k_scale=ks, v_scale=vs,
                                          window=w)
        for part in (0, 16, 128):
            out, lse = gu.decode(dp, 0, q_dev, tdev, lens, hq, part, q_dtype=qdt, window=w)
            gu.assert_close(out.cpu().numpy(), ref, "out w=%d part=%d" % (w, part))
            gu.assert_close(lse.cpu().numpy(), ref_lse, "lse w=%d part=%d" % (w, part))


def test_trimmed_growing_sequence_ignores_reused_blocks():
    import torch
    import paged_kv_cache_inject_amd as pkv
    from oracle import attention as o_att, inject as o_inject
    from oracle.allocator import AllocatorModel
    from oracle.rope import rope_table
    from tests import gpu_util as gu
    from workloads.configs import host_normal

    rng = np.random.default_rng(11)
    H, d, HQ, NB, W, MB = 2, 128, 8, 10, 60, 64
    max_pos = 1024
    dp = gu.DevicePool(1, NB, H, d, "bf16", fill_bits=0x7FC1)     # NaN canaries
    cache = pkv.pkv_cache_create(NB, 2, MB, free_list_seed=4)
    model = AllocatorModel(NB, 2, MB, seed=4)
    ref = np.full(dp.total, 0x7FC1, dtype=np.uint16)
    kp, vp = dp.oracle_arrays(ref)
    o_cos, o_sin = rope_table(d, 10000.0, max_pos)
    _, _, dcos, dsin = gu.rope_tables(d, max_pos)
    keep = []
    nan16 = np.full((1, 1, H, d), 0x7FC1, dtype=np.uint16)

    def append(seq, n, values=None):
        first = list(pkv.pkv_extend(cache, [seq], n))
        assert first == model.extend([seq], n)
        table, _ = pkv.pkv_block_table(cache, [seq], MB)
        tdev = torch.from_numpy(table).cuda()
        fdev = torch.from_numpy(np.asarray(first, np.int32)).cuda()
        k_new = host_normal(rng, (1, n, H, d), "bf16") if values is None else values
        v_new = host_normal(rng, (1, n, H, d), "bf16") if values is None else values
        kd = gu.to_device_raw(k_new.reshape(-1), "bf16")
        vd = gu.to_device_raw(v_new.reshape(-1), "bf16")
        keep.append((kd, vd, tdev, fdev))
        pkv.pkv_append_kv(dp.desc(), 0, tdev, fdev, n, kd, vd, "pairs", dcos, dsin, max_pos)
        o_inject.append(kp, vp, dp.spec(), 0, model.tables, model.lens, [seq], n, k_new, v_new,
                        "pairs", o_cos, o_sin)

    crng = np.random.default_rng(12)                       # step sizes
    for step in range(30):
        append(0, int(crng.choice([1, 3, 16])))
        assert pkv.pkv_trim_window(cache, [0], W) == model.trim_window([0], W)
        if step % 5 == 4 and pkv.pkv_num_free_blocks(cache) > 0:
            append(1, 1, values=nan16)                         # takes a dropped block
    # A NaN token inside the window's first block but before the window:
    # bring the length to 2 past a block boundary, write NaN there, then 65
    # more tokens, so that the window starts 6 positions after it.
    append(0, (2 - model.lens[0]) % 16 or 16)
    assert pkv.pkv_trim_window(cache, [0], W) == model.trim_window([0], W)
    nan_pos = model.lens[0]
    append(0, 1, values=nan16)
    append(0, 65)
    assert pkv.pkv_trim_window(cache, [0], W) == model.trim_window([0], W)
    lo = model.lens[0] - W
    assert nan_pos < lo and nan_pos // 16 == lo // 16 and model.tables[0][lo // 16] >= 0
    held = sum(1 for b in model.tables[0] if b >= 0)
    assert held <= -(-W // 16) + 1 and model.lens[0] > 2 * W
    torch.cuda.synchronize()
    gu.assert_bytes_equal(dp.host_copy(), ref, "pool after appends and trims")
    table, lens = pkv.pkv_block_table(cache, [0], MB)
    q = host_normal(rng, (1, HQ, d), "bf16")
    q_dev = gu.to_device_raw(q.reshape(-1), "bf16").view(1, HQ, d)
    r_out, r_lse = o_att.decode_paged(q, kp, vp, dp.spec(), 0, [model.tables[0]], lens, HQ,
                                      by_plane=True, window=W)
    for part in (0, 16):
        out, lse = gu.decode(dp, 0, q_dev, torch.from_numpy(table).cuda(), lens, HQ, part,
                             window=W)
        assert np.isfinite(out.cpu().numpy()).all()
        gu.assert_close(out.cpu().numpy(), r_out, "trimmed out part=%d" % part)
        gu.assert_close(lse.cpu().numpy(), r_lse, "trimmed lse part=%d" % part)
    # writes into dropped positions are refused before anything is enqueued
    src_t = torch.zeros(64 * H * d, dtype=torch.bfloat16, device="cuda")
    src = pkv.make_src(src_t, src_t, 0, H * d, 64)
    ws = gu.workspace(1 << 16)
    with pytest.raises(pkv.PkvError) as e:
        pkv.pkv_inject(cache, dp.desc(), src, [(0, 4, 0, 0)], 0, 1, "pairs", dcos, dsin,
                       max_pos, ws)
    assert e.value.code == "RANGE"
    pkv.pkv_cache_destroy(cache)
