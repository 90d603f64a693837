"""The quantised (fp8 E4M3) cache on the GPU against the oracle: inject and
append byte for byte (rotation in float32, division by the per-(layer, KV
head) scale, round to nearest even with saturation), and decode within
tolerance of the oracle's float64 attention over the dequantised values."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def scales(rng, L, H, nb=None):
    """Scales per (layer, KV head), or per (layer, block, KV head) when nb is
    given (pool scale_mode 1)."""
    shape = (L, H) if nb is None else (L, nb, H)
    k = rng.uniform(0.004, 0.03, size=shape).astype(np.float32)
    v = rng.uniform(0.004, 0.03, size=shape).astype(np.float32)
    return k, v


@pytest.mark.parametrize("sdt,d,mode,blockwise", [
    ("bf16", 128, "pairs", False), ("bf16", 128, "halves", False), ("f16", 64, "pairs", False),
    ("bf16", 64, "none", False), ("bf16", 128, "pairs", True), ("f16", 64, "halves", True)])
def test_fp8_inject_matches_oracle(sdt, d, mode, blockwise):
    import torch
    import paged_kv_cache_inject_amd as pkv
    from oracle import inject as o_inject
    from oracle.allocator import AllocatorModel
    from oracle.rope import rope_table
    from tests import gpu_util as gu
    from workloads.configs import host_normal

    gu.say("fp8 inject", sdt, d, mode, "per block" if blockwise else "per head")
    rng = np.random.default_rng(hash((sdt, d, mode, blockwise)) % 2 ** 32)
    L, H, NB, max_pos = 3, 4, 48, 300
    dp = gu.DevicePool(L, NB, H, d, "fp8", fill_bits=0x5A)
    ks, vs = scales(rng, L, H, NB if blockwise else None)
    dp.set_scales(ks, vs)
    cache = pkv.pkv_cache_create(NB, 4, 16, free_list_seed=21)
    model = AllocatorModel(NB, 4, 16, seed=21)
    for s, n in enumerate((100, 37, 250, 16)):
        pkv.pkv_alloc_blocks(cache, s, n)
        model.alloc_blocks(s, n)
    n_src = 400
    src_k = host_normal(rng, (L, n_src, H, d), sdt)
    src_v = host_normal(rng, (L, n_src, H, d), sdt)
    calls = [[(0, 100, 0, 0), (1, 37, 0, 100), (3, 16, 0, 137)],
             [(2, 5, 3, 200), (2, 40, 9, 153), (2, 100, 60, 210), (0, 24, 40, 300)]]
    o_cos, o_sin = rope_table(d, 10000.0, max_pos)
    _, _, dcos, dsin = gu.rope_tables(d, max_pos)
    dk = gu.to_device_raw(src_k.reshape(-1), sdt)
    dv = gu.to_device_raw(src_v.reshape(-1), sdt)
    src = pkv.make_src(dk, dv, n_src * H * d, H * d, n_src, dtype=sdt)
    ref = np.full(dp.total, 0x5A, dtype=np.uint8)
    kp, vp = dp.oracle_arrays(ref)
    lens = [0] * 4
    for i, runs in enumerate(calls):
        ws = gu.workspace(pkv.pkv_inject_workspace_bytes(runs))
        pkv.pkv_inject(cache, dp.desc(), src, runs, 0, L, mode, dcos, dsin, max_pos, ws)
        torch.cuda.synchronize()
        lens = o_inject.inject(kp, vp, dp.spec(), model.tables, lens, runs, src_k.reshape(-1),
                               src_v.reshape(-1), n_src * H * d, H * d, 0, L, mode, o_cos, o_sin,
                               src_dtype=sdt, k_scale=ks, v_scale=vs)
        gu.assert_bytes_equal(dp.host_copy(), ref, "fp8 pool after inject call %d" % i)


@pytest.mark.parametrize("sdt,n_new,blockwise", [("bf16", 1, False), ("bf16", 17, False),
                                                 ("f16", 32, False), ("bf16", 17, True)])
def test_fp8_append_matches_oracle(sdt, n_new, blockwise):
    import torch
    import paged_kv_cache_inject_amd as pkv
    from oracle import inject as o_inject
    from oracle.allocator import AllocatorModel
    from oracle.rope import rope_table
    from tests import gpu_util as gu
    from workloads.configs import host_normal

    rng = np.random.default_rng(n_new + 100 + blockwise)
    L, H, NB, B, d, max_pos = 2, 8, 64, 6, 128, 512
    dp = gu.DevicePool(L, NB, H, d, "fp8", fill_bits=0x33)
    ks, vs = scales(rng, L, H, NB if blockwise else None)
    dp.set_scales(ks, vs)
    cache = pkv.pkv_cache_create(NB, B, 32, free_list_seed=5)
    model = AllocatorModel(NB, B, 32, seed=5)
    for s, n in enumerate([0, 15, 16, 31, 100, 47]):
        pkv.pkv_extend(cache, [s], n)
        model.extend([s], n)
    seqs = list(range(B))
    first = pkv.pkv_extend(cache, seqs, n_new)
    assert list(first) == model.extend(seqs, n_new)
    table, _ = pkv.pkv_block_table(cache, seqs, 32)
    o_cos, o_sin = rope_table(d, 10000.0, max_pos)
    _, _, dcos, dsin = gu.rope_tables(d, max_pos)
    ref = np.full(dp.total, 0x33, dtype=np.uint8)
    kp, vp = dp.oracle_arrays(ref)
    tdev = torch.from_numpy(table).cuda()
    fdev = torch.from_numpy(first.astype(np.int32)).cuda()
    keep = []
    for layer in range(L):
        k_new = host_normal(rng, (B, n_new, H, d), sdt)
        v_new = host_normal(rng, (B, n_new, H, d), sdt)
        kd = gu.to_device_raw(k_new.reshape(-1), sdt)
        vd = gu.to_device_raw(v_new.reshape(-1), sdt)
        keep.append((kd, vd))
        pkv.pkv_append_kv(dp.desc(), layer, tdev, fdev, n_new, kd, vd, "pairs", dcos, dsin,
                          max_pos, new_dtype=sdt)
        o_inject.append(kp, vp, dp.spec(), layer, model.tables, model.lens, seqs, n_new,
                        k_new, v_new, "pairs", o_cos, o_sin, src_dtype=sdt, k_scale=ks,
                        v_scale=vs)
    torch.cuda.synchronize()
    gu.assert_bytes_equal(dp.host_copy(), ref, "fp8 pool after append")


@pytest.mark.parametrize("qdt,hq,hkv,d,blockwise", [
    ("bf16", 64, 8, 128, False), ("f16", 32, 8, 128, False), ("bf16", 8, 8, 128, False),
    ("bf16", 16, 2, 64, False), ("bf16", 64, 2, 128, False), ("f16", 64, 1, 64, False),
    ("bf16", 64, 8, 128, True), ("f16", 64, 1, 64, True), ("bf16", 32, 2, 128, True)])
def test_fp8_decode_matches_oracle(qdt, hq, hkv, d, blockwise):
    import torch
    from oracle import attention as o_att
    from tests import gpu_util as gu
    from workloads.configs import host_normal, deal_tables

    rng = np.random.default_rng(hq * 7 + hkv + d)
    lens = np.array([1, 15, 16, 17, 0, 33, 200, 700, 2000], dtype=np.int64)
    need = int(sum(-(-x // 16) for x in lens))
    nb = need + 5
    table = deal_tables(rng.permutation(nb)[:need].astype(np.int32), lens, 128)
    dp = gu.DevicePool(1, nb, hkv, d, "fp8")
    ks, vs = scales(rng, 1, hkv, nb if blockwise else None)
    dp.set_scales(ks, vs)
    # codes of magnitude up to ~448 times scales ~0.01: values of order 1
    codes = rng.integers(0, 0x7F, size=dp.total, dtype=np.uint8)
    codes |= (rng.integers(0, 2, size=dp.total, dtype=np.uint8) << 7).astype(np.uint8)
    codes = np.where((codes & 0x7F) > 0x5F, codes & 0xDF, codes).astype(np.uint8)  # |x| <~ 16
    dp.buf.copy_(gu.to_device_raw(codes, "fp8"))
    q = host_normal(rng, (len(lens), hq, d), qdt)
    kp, vp = dp.oracle_arrays(codes)
    ref, ref_lse = o_att.decode_paged(q, kp, vp, dp.spec(), 0, [list(r) for r in table], lens,
                                      hq, by_plane=True, q_dtype=qdt, k_scale=ks, v_scale=vs)
    q_dev = gu.to_device_raw(q.reshape(-1), qdt).view(q.shape)
    tdev = torch.from_numpy(table).cuda()
    for part in (0, 16, 256):
        out, lse = gu.decode(dp, 0, q_dev, tdev, lens, hq, part, q_dtype=qdt)
        gu.assert_close(out.cpu().numpy(), ref, "fp8 out part=%d" % part)
        gu.assert_close(lse.cpu().numpy(), ref_lse, "fp8 lse part=%d" % part)


def test_fp8_inject_then_decode_tracks_bf16_path():
    """The same stored chunk injected into a bf16 and an fp8 pool: decode
    outputs differ only by the fp8 rounding of K and V (a few percent)."""
    import torch
    import paged_kv_cache_inject_amd as pkv
    from tests import gpu_util as gu
    from workloads.configs import host_normal

    rng = np.random.default_rng(77)
    d, H, HQ, n = 128, 8, 32, 600
    max_pos = 1024
    src_k = host_normal(rng, (1, n, H, d), "bf16")
    src_v = host_normal(rng, (1, n, H, d), "bf16")
    dk = gu.to_device_raw(src_k.reshape(-1), "bf16")
    dv = gu.to_device_raw(src_v.reshape(-1), "bf16")
    _, _, dcos, dsin = gu.rope_tables(d, max_pos)
    q = host_normal(rng, (1, HQ, d), "bf16")
    q_dev = gu.to_device_raw(q.reshape(-1), "bf16").view(1, HQ, d)
    outs = []
    for dtype in ("bf16", "fp8"):
        nb = 48
        dp = gu.DevicePool(1, nb, H, d, dtype, fill_bits=0)
        if dtype == "fp8":
            amax = 4.5
            dp.set_scales(np.full((1, H), amax / 448, np.float32), np.full((1, H), amax / 448, np.float32))
        cache = pkv.pkv_cache_create(nb, 1, nb)
        pkv.pkv_alloc_blocks(cache, 0, n)
        src = pkv.make_src(dk, dv, 0, H * d, n, dtype="bf16")
        ws = gu.workspace(pkv.pkv_inject_workspace_bytes([(0, n, 0, 0)]))
        pkv.pkv_inject(cache, dp.desc(), src, [(0, n, 0, 0)], 0, 1, "pairs", dcos, dsin, max_pos, ws)
        table, lens = pkv.pkv_block_table(cache, [0], nb)
        out, _ = gu.decode(dp, 0, q_dev, torch.from_numpy(table).cuda(), lens, HQ, 0,
                           q_dtype="bf16")
        outs.append(out.cpu().numpy())
        pkv.pkv_cache_destroy(cache)
    err = np.abs(outs[0] - outs[1])
    assert np.max(err) < 0.05 and np.mean(err) < 0.01, (np.max(err), np.mean(err))


def test_fp8_nan_codes_in_unused_slots_do_not_leak():
    """Slots past each sequence's end and blocks no table names hold the NaN
    code; the decode output depends only on the live slots."""
    import torch
    from oracle import attention as o_att
    from oracle.layout import k_element_offsets, v_element_offsets
    from tests import gpu_util as gu
    from workloads.configs import host_normal, deal_tables

    rng = np.random.default_rng(4242)
    hq, hkv, d = 32, 8, 128
    lens = np.array([1, 15, 17, 31, 300, 0, 129], dtype=np.int64)
    need = int(sum(-(-x // 16) for x in lens))
    nb = need + 3
    table = deal_tables(rng.permutation(nb)[:need].astype(np.int32), lens, 32)
    dp = gu.DevicePool(1, nb, hkv, d, "fp8")
    ks, vs = scales(rng, 1, hkv)
    dp.set_scales(ks, vs)
    codes = rng.integers(0, 0x60, size=dp.total, dtype=np.uint8)
    codes |= (rng.integers(0, 2, size=dp.total, dtype=np.uint8) << 7).astype(np.uint8)
    live = np.zeros(dp.total, dtype=bool)
    kp, vp = dp.oracle_arrays(codes)
    spec = dp.spec()
    for b, n in enumerate(lens):
        for p in range(int(n)):
            blk = int(table[b][p // 16])
            for h in range(hkv):
                live[k_element_offsets(spec, 0, blk, h, p % 16)] = True
                live[dp.v_off + v_element_offsets(spec, 0, blk, h, p % 16)] = True
    codes[~live] = np.where(rng.integers(0, 2, size=int((~live).sum())) == 1, 0xFF, 0x7F)
    dp.buf.copy_(gu.to_device_raw(codes, "fp8"))
    q = host_normal(rng, (len(lens), hq, d), "bf16")
    ref, ref_lse = o_att.decode_paged(q, kp, vp, spec, 0, [list(r) for r in table], lens, hq,
                                      by_plane=True, q_dtype="bf16", k_scale=ks, v_scale=vs)
    assert np.all(np.isfinite(ref))
    q_dev = gu.to_device_raw(q.reshape(-1), "bf16").view(q.shape)
    tdev = torch.from_numpy(table).cuda()
    for part in (0, 16, 64):
        out, lse = gu.decode(dp, 0, q_dev, tdev, lens, hq, part, q_dtype="bf16")
        gu.assert_close(out.cpu().numpy(), ref, "fp8 NaN-canary out part=%d" % part)
        gu.assert_close(lse.cpu().numpy(), ref_lse, "fp8 NaN-canary lse part=%d" % part)


def test_fp8_block_copy_carries_per_block_scales():
    """Copy-on-write of a block of an fp8 pool with scales per (layer, block,
    KV head): pkv_copy_blocks copies the planes and the block's scale
    entries, as the oracle's copy does; other entries keep their values."""
    import torch
    import paged_kv_cache_inject_amd as pkv
    from oracle import inject as o_inject
    from tests import gpu_util as gu

    rng = np.random.default_rng(808)
    L, H, NB, d = 3, 4, 12, 128
    dp = gu.DevicePool(L, NB, H, d, "fp8")
    ks, vs = scales(rng, L, H, NB)
    dp.set_scales(ks, vs)
    codes = rng.integers(0, 0x7E, size=dp.total, dtype=np.uint8)
    dp.buf.copy_(gu.to_device_raw(codes, "fp8"))
    cache = pkv.pkv_cache_create(NB, 2, 8, free_list_seed=4)
    pkv.pkv_extend(cache, [0], 20)                  # two blocks
    pkv.pkv_fork(cache, 0, 1)
    pkv.pkv_extend(cache, [1], 1)                   # position 20 lies in the shared block
    pairs = [tuple(int(x) for x in pr) for pr in pkv.pkv_pending_copies(cache)]
    assert len(pairs) == 1
    pkv.pkv_copy_blocks(cache, dp.desc())
    torch.cuda.synchronize()
    ref = codes.copy()
    kp, vp = dp.oracle_arrays(ref)
    k_ref, v_ref = ks.copy(), vs.copy()
    o_inject.copy_blocks(kp, vp, dp.spec(), pairs, k_scale=k_ref, v_scale=v_ref)
    gu.assert_bytes_equal(dp.host_copy(), ref, "fp8 pool after the copy")
    assert np.array_equal(dp.k_scale.cpu().numpy(), k_ref)
    assert np.array_equal(dp.v_scale.cpu().numpy(), v_ref)
    src, dst = pairs[0]
    assert np.array_equal(k_ref[:, dst], ks[:, src]) and not np.array_equal(ks[:, dst], ks[:, src])
    pkv.pkv_cache_destroy(cache)


@pytest.mark.parametrize("sdt", ["bf16", "f16"])
def test_fp8_encoding_of_every_16bit_value(sdt):
    """Every bf16 (or f16) bit pattern -- zeros, subnormals, values around
    the E4M3 ties and the 448 saturation point, infinities, NaNs -- injected
    unrotated into an fp8 pool with unit scales: the stored codes equal the
    oracle's round-to-nearest-even, saturating encoding byte for byte."""
    import torch
    import paged_kv_cache_inject_amd as pkv
    from oracle import inject as o_inject
    from oracle.allocator import AllocatorModel
    from oracle.rope import rope_table
    from tests import gpu_util as gu

    L, H, d = 1, 1, 64
    n_tok = 65536 // (H * d)                      # 1,024 tokens hold every pattern once
    NB = n_tok // 16
    dp = gu.DevicePool(L, NB, H, d, "fp8", fill_bits=0x11)
    ks = np.ones((L, H), np.float32)
    dp.set_scales(ks, ks)
    pat = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    src_k = pat.reshape(L, n_tok, H, d)
    src_v = pat[::-1].copy().reshape(L, n_tok, H, d)
    cache = pkv.pkv_cache_create(NB, 1, NB, free_list_seed=2)
    model = AllocatorModel(NB, 1, NB, seed=2)
    pkv.pkv_alloc_blocks(cache, 0, n_tok)
    model.alloc_blocks(0, n_tok)
    dk = gu.to_device_raw(src_k.reshape(-1), sdt)
    dv = gu.to_device_raw(src_v.reshape(-1), sdt)
    src = pkv.make_src(dk, dv, n_tok * H * d, H * d, n_tok, dtype=sdt)
    runs = [(0, n_tok, 0, 0)]
    ws = gu.workspace(pkv.pkv_inject_workspace_bytes(runs))
    o_cos, o_sin = rope_table(d, 10000.0, n_tok)
    _, _, dcos, dsin = gu.rope_tables(d, n_tok)
    pkv.pkv_inject(cache, dp.desc(), src, runs, 0, L, "none", dcos, dsin, n_tok, ws)
    torch.cuda.synchronize()
    ref = np.full(dp.total, 0x11, dtype=np.uint8)
    kp, vp = dp.oracle_arrays(ref)
    o_inject.inject(kp, vp, dp.spec(), model.tables, [0], runs, src_k.reshape(-1),
                    src_v.reshape(-1), n_tok * H * d, H * d, 0, L, "none", o_cos, o_sin,
                    src_dtype=sdt, k_scale=ks, v_scale=ks)
    gu.assert_bytes_equal(dp.host_copy(), ref, "fp8 codes of every %s value" % sdt)
    pkv.pkv_cache_destroy(cache)
