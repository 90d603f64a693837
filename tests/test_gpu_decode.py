"""Read side on the GPU against the oracle: decode attention for the
Llama-3-8B-shaped layer in full, edge lengths and split sizes, bit-identity
under physical-block permutation, Theorem 1 (relocated keys), and sampled
outputs of the full-size ragged MHA and Llama-3-70B-shaped workloads."""

import os

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def fill_random_pool(dp, seed):
    """N(0,1) values in every element of the pool, drawn on the device."""
    from workloads.configs import device_normal
    for layer in range(dp.n_layers):
        a, b = layer * dp.layer_stride, (layer + 1) * dp.layer_stride
        dp.buf[a:b] = device_normal(b - a, dp.dtype, seed * 1000 + layer)


def check_decode_all(dp, layer, q_raw, table, lens, hq, parts=(0,), variants=("auto",),
                     seqs=None):
    import torch
    from oracle import attention as o_att
    from tests import gpu_util as gu
    flat = dp.host_copy() if seqs is None else gu.host_planes_for(dp, layer, table, seqs, None)
    kp, vp = dp.oracle_arrays(flat)
    rows = [list(r) for r in table]
    ref, ref_lse = o_att.decode_paged(q_raw, kp, vp, dp.spec(), layer, rows, lens, hq,
                                      seqs=seqs, by_plane=True)
    q_dev = gu.to_device_raw(q_raw.reshape(-1), dp.dtype).view(q_raw.shape)
    tables_dev = torch.from_numpy(np.ascontiguousarray(table, dtype=np.int32)).cuda()
    worst = 0.0
    sel = slice(None) if seqs is None else list(seqs)
    for variant in variants:
        if variant == "valu":
            os.environ["PKV_DECODE_KERNEL"] = "1"
        elif variant == "dot2":
            os.environ["PKV_DECODE_KERNEL"] = "2"
        elif variant == "staged":
            os.environ["PKV_DECODE_KERNEL"] = "12"
        try:
            for part in parts:
                out, lse = gu.decode(dp, layer, q_dev, tables_dev, lens, hq, part)
                o, l = out.cpu().numpy(), lse.cpu().numpy()
                worst = max(worst, gu.assert_close(o[sel], ref[sel], "out %s part=%d" % (variant, part)))
                gu.assert_close(l[sel], ref_lse[sel], "lse %s part=%d" % (variant, part))
        finally:
            os.environ.pop("PKV_DECODE_KERNEL", None)
    return worst


def test_llama8b_layer_full():
    from tests import gpu_util as gu
    from workloads.configs import LLAMA8B_1LAYER, llama8b_structure, host_normal
    cfg = LLAMA8B_1LAYER
    st = llama8b_structure(cfg)
    gu.say("llama8b decode: pool", st["num_blocks"], "blocks, sum len", int(st["lens"].sum()))
    dp = gu.DevicePool(1, st["num_blocks"], cfg.n_kv_heads, cfg.head_dim, cfg.dtype)
    fill_random_pool(dp, cfg.seed)
    q = host_normal(st["rng"], (cfg.batch, cfg.n_q_heads, cfg.head_dim), cfg.dtype)
    worst = check_decode_all(dp, 0, q, st["tables"], st["lens"], cfg.n_q_heads,
                             parts=(0, 256, 1024), variants=("auto", "valu"))
    gu.say("llama8b worst abs err", worst)


@pytest.mark.parametrize("dtype,hq,hkv,d", [
    ("bf16", 64, 8, 128), ("bf16", 32, 8, 128), ("f16", 8, 8, 128), ("bf16", 16, 1, 64),
    ("f16", 32, 2, 64), ("f32", 4, 2, 64), ("bf16", 6, 2, 128),
    # more than 16 query heads per KV head: 2 or 4 tiles of 16, the last one partial
    ("bf16", 32, 1, 128), ("f16", 48, 2, 64), ("bf16", 64, 1, 128), ("f16", 40, 1, 64),
])
def test_edge_lengths_and_splits(dtype, hq, hkv, d):
    from tests import gpu_util as gu
    from workloads.configs import host_normal, deal_tables
    rng = np.random.default_rng(hq * 131 + hkv * 7 + d)
    lens = np.array([1, 15, 16, 17, 0, 33, 64, 200, 5, 1000], dtype=np.int64)
    need = int(sum(-(-x // 16) for x in lens))
    nb = need + 7
    ids = rng.permutation(nb)[:need].astype(np.int32)
    table = deal_tables(ids, lens, 64)
    dp = gu.DevicePool(1, nb, hkv, d, dtype)
    fill_random_pool(dp, 17)
    q = host_normal(rng, (len(lens), hq, d), dtype)
    check_decode_all(dp, 0, q, table, lens, hq, parts=(0, 16, 48, 256),
                     variants=("auto", "valu"))


def test_peaky_scores():
    """Large query norms make the softmax nearly one-hot (stress for the
    rescaling and the 16-bit probability split)."""
    import torch
    from tests import gpu_util as gu
    from workloads.configs import host_normal, deal_tables
    from oracle.numerics import f32_to_bf16_rne, to_f32
    rng = np.random.default_rng(99)
    lens = np.array([3, 40, 700, 2000], dtype=np.int64)
    need = int(sum(-(-x // 16) for x in lens))
    table = deal_tables(rng.permutation(need).astype(np.int32), lens, 128)
    dp = gu.DevicePool(1, need, 8, 128, "bf16")
    fill_random_pool(dp, 23)
    q = f32_to_bf16_rne(to_f32(host_normal(rng, (4, 64, 128), "bf16"), "bf16") * 8.0)
    check_decode_all(dp, 0, q, table, lens, 64, parts=(0, 32, 512), variants=("auto", "valu"))


def test_block_permutation_gives_identical_bits():
    """The same logical K/V under two physical placements: bit-identical output."""
    import torch
    from tests import gpu_util as gu
    from workloads.configs import host_normal
    rng = np.random.default_rng(5)
    lens = np.array([700, 33, 1024, 250], dtype=np.int64)
    nblk = [-(-int(x) // 16) for x in lens]
    need = sum(nblk)
    hkv, d, hq = 8, 128, 64
    pools, tables = [], []
    logical = host_normal(rng, (need, 2 * hkv * 16 * d), "bf16")   # one row per logical block
    for perm_seed in (1, 2):
        perm = np.random.default_rng(perm_seed).permutation(need)
        dp = gu.DevicePool(1, need, hkv, d, "bf16")
        host = np.empty((need, 2 * hkv * 16 * d), np.uint16)
        host[perm] = logical                  # logical block i -> physical perm[i]
        dp.buf.copy_(gu.to_device_raw(host.reshape(-1), "bf16"))
        table = np.full((4, 64), -1, np.int32)
        at = 0
        for b, n in enumerate(nblk):
            table[b, :n] = perm[at:at + n]
            at += n
        pools.append(dp)
        tables.append(table)
    q = host_normal(rng, (4, hq, d), "bf16")
    q_dev = gu.to_device_raw(q.reshape(-1), "bf16").view(4, hq, d)
    outs = []
    for dp, table in zip(pools, tables):
        out, lse = gu.decode(dp, 0, q_dev, torch.from_numpy(table).cuda(), lens, hq, 256)
        outs.append((out.cpu().numpy(), lse.cpu().numpy()))
    assert np.array_equal(outs[0][0].view(np.uint32), outs[1][0].view(np.uint32))
    assert np.array_equal(outs[0][1].view(np.uint32), outs[1][1].view(np.uint32))


def test_theorem1_inject_equals_relative_form():
    """Keys rotated at insert (inject) and keys rotated before insert
    (append, rotation off) both score by relative position only."""
    import torch
    import paged_kv_cache_inject_amd as pkv
    from oracle import attention as o_att
    from oracle.rope import rope_matrix
    from tests import gpu_util as gu
    rng = np.random.default_rng(31)
    d, hq, hkv, n, p0, m = 128, 8, 2, 90, 13, 150
    max_pos = 256
    k_pre = rng.standard_normal((n, hkv, d)).astype(np.float32)
    v = rng.standard_normal((n, hkv, d)).astype(np.float32)
    q_pre = rng.standard_normal((1, hq, d))
    q_rot = np.stack([rope_matrix(m, d, 10000.0) @ q_pre[0, h] for h in range(hq)])[None]
    _, _, dcos, dsin = gu.rope_tables(d, max_pos)
    results = []
    for path in ("inject", "prerotated"):
        nb = 8
        dp = gu.DevicePool(1, nb, hkv, d, "f32", fill_bits=0)
        cache = pkv.pkv_cache_create(nb, 1, nb)
        pkv.pkv_alloc_blocks(cache, 0, p0 + n)
        table, _ = pkv.pkv_block_table(cache, [0], nb)
        tdev = torch.from_numpy(table).cuda()
        if path == "inject":
            sk = torch.from_numpy(k_pre.reshape(-1)).cuda()
            sv = torch.from_numpy(v.reshape(-1)).cuda()
            src = pkv.make_src(sk, sv, 0, hkv * d, n)
            ws = gu.workspace(pkv.pkv_inject_workspace_bytes([(0, n, p0, 0)]))
            pkv.pkv_inject(cache, dp.desc(), src, [(0, n, p0, 0)], 0, 1, "pairs", dcos, dsin,
                           max_pos, ws)
        else:
            rot = np.stack([[rope_matrix(p0 + t, d, 10000.0) @ k_pre[t, h].astype(np.float64)
                             for h in range(hkv)] for t in range(n)]).astype(np.float32)
            first = torch.tensor([p0], dtype=torch.int32, device="cuda")
            pkv.pkv_append_kv(dp.desc(), 0, tdev, first, n,
                              torch.from_numpy(rot.reshape(-1)).cuda(),
                              torch.from_numpy(v.reshape(-1)).cuda(), "none", None, None, 0)
        torch.cuda.synchronize()
        # attend over positions p0 .. p0+n-1 only: shift the table so they
        # start a fresh sequence is not possible (p0 unaligned), so positions
        # below p0 hold zeros (keys 0 -> score 0, values 0) and are accounted
        # for in the reference below.
        q_dev = torch.from_numpy(q_rot.astype(np.float32).reshape(-1)).cuda().view(1, hq, d)
        out, lse = gu.decode(dp, 0, q_dev, tdev, np.array([p0 + n]), hq, 0)
        results.append(out.cpu().numpy())
        pkv.pkv_cache_destroy(cache)
    g = hq // hkv
    ref = np.zeros((1, hq, d))
    for h in range(hq):
        rel = np.stack([rope_matrix(p0 + t - m, d, 10000.0) @ k_pre[t, h // g].astype(np.float64)
                        for t in range(n)])
        k_all = np.concatenate([np.zeros((p0, d)), rel])
        v_all = np.concatenate([np.zeros((p0, d)), v[:, h // g].astype(np.float64)])
        ref[0, h], _ = o_att.softmax_attend(q_pre[0, h], k_all, v_all, d ** -0.5)
    from tests import gpu_util as gu2
    gu2.assert_close(results[0], ref, "inject path vs relative form")
    gu2.assert_close(results[1], ref, "pre-rotated path vs relative form")
    gu2.assert_close(results[0], results[1], "inject vs pre-rotated", atol=1e-5, rtol=1e-5)


def test_ragged_mha_full_size_sampled():
    import torch
    from tests import gpu_util as gu
    from workloads.configs import RAGGED_MHA, ragged_mha_structure, host_normal
    cfg = RAGGED_MHA
    st = ragged_mha_structure(cfg)
    lens = st["lens"]
    gu.say("ragged MHA: pool", st["num_blocks"], "blocks, max len", int(lens.max()))
    dp = gu.DevicePool(1, st["num_blocks"], cfg.n_kv_heads, cfg.head_dim, cfg.dtype)
    fill_random_pool(dp, cfg.seed)
    q = host_normal(st["rng"], (cfg.batch, cfg.n_q_heads, cfg.head_dim), cfg.dtype)
    order = np.argsort(lens)
    seqs = sorted(set(order[:6].tolist() + order[-6:].tolist() +
                      np.random.default_rng(0).choice(cfg.batch, 12, replace=False).tolist()))
    check_decode_all(dp, 0, q, st["tables"], lens, cfg.n_q_heads, parts=(0,), seqs=seqs)


def test_llama70b_full_size_sampled():
    import torch
    from tests import gpu_util as gu
    from workloads.configs import LLAMA70B_80LAYER, llama70b_structure, host_normal
    cfg = LLAMA70B_80LAYER
    st = llama70b_structure(cfg)
    gu.say("llama70b: 80 layers x", st["num_blocks"], "blocks")
    dp = gu.DevicePool(cfg.n_layers, st["num_blocks"], cfg.n_kv_heads, cfg.head_dim, cfg.dtype)
    fill_random_pool(dp, cfg.seed)
    q = host_normal(st["rng"], (cfg.batch, cfg.n_q_heads, cfg.head_dim), cfg.dtype)
    for layer in (0, 41, 79):
        seqs = np.random.default_rng(layer).choice(cfg.batch, 3, replace=False).tolist()
        check_decode_all(dp, layer, q, st["tables"], st["lens"], cfg.n_q_heads, parts=(0,),
                         seqs=seqs)
    del dp
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype,hq,hkv,d", [("bf16", 64, 8, 128), ("f16", 8, 8, 128),
                                             ("f32", 4, 2, 64), ("bf16", 4, 2, 64)])
def test_nan_in_unused_slots_does_not_leak(dtype, hq, hkv, d):
    """Slots past a sequence's end hold NaN; the output must not see them."""
    import torch
    from oracle.layout import k_element_offsets, v_element_offsets
    from tests import gpu_util as gu
    from workloads.configs import host_normal, deal_tables
    rng = np.random.default_rng(41)
    lens = np.array([1, 17, 30, 100, 250], dtype=np.int64)
    need = int(sum(-(-x // 16) for x in lens))
    table = deal_tables(rng.permutation(need).astype(np.int32), lens, 16)
    dp = gu.DevicePool(1, need, hkv, d, dtype)
    host = host_normal(rng, (dp.total,), dtype)
    nan = np.float32(np.nan) if dtype == "f32" else np.uint16(0x7FC1 if dtype == "bf16" else 0x7E01)
    kp, vp = dp.oracle_arrays(host)
    for b, n in enumerate(lens):
        blk = table[b][(n - 1) // 16]
        for t in range(int(n) % 16 or 16, 16):
            for h in range(hkv):
                kp[k_element_offsets(dp.spec(), 0, blk, h, t)] = nan
                vp[v_element_offsets(dp.spec(), 0, blk, h, t)] = nan
    dp.buf.copy_(gu.to_device_raw(host, dtype))
    q = host_normal(rng, (len(lens), hq, d), dtype)
    check_decode_all(dp, 0, q, table, lens, hq, parts=(0, 16, 64), variants=("auto", "valu"))


@pytest.mark.parametrize("dtype,hq,hkv,d", [("bf16", 64, 8, 64), ("bf16", 32, 1, 64),
                                             ("f16", 16, 2, 128), ("bf16", 16, 8, 128)])
def test_eight_wave_launches_with_one_workgroup_per_cu(dtype, hq, hkv, d):
    """Sequences long enough for 8-wave workgroups, few workgroups per CU:
    these launches ask for extra dynamic LDS (one workgroup per CU), up to
    ~47 KB of it at d = 64.  One and two tiles of query heads."""
    from workloads.configs import host_normal, deal_tables
    from tests import gpu_util as gu
    rng = np.random.default_rng(hq + hkv + d)
    lens = np.array([600, 1500, 2047, 900, 3000], dtype=np.int64)
    need = int(sum(-(-x // 16) for x in lens))
    table = deal_tables(rng.permutation(need + 3)[:need].astype(np.int32), lens, 256)
    dp = gu.DevicePool(1, need + 3, hkv, d, dtype)
    fill_random_pool(dp, 29)
    q = host_normal(rng, (len(lens), hq, d), dtype)
    check_decode_all(dp, 0, q, table, lens, hq, parts=(0, 512))


@pytest.mark.parametrize("dtype,hq,hkv,d", [("bf16", 32, 8, 128), ("f16", 8, 8, 128),
                                             ("bf16", 6, 2, 64), ("f16", 12, 4, 64),
                                             ("bf16", 8, 4, 128)])
def test_dot2_kernel_small_groups(dtype, hq, hkv, d):
    """The packed-dot-product kernel (query groups of 1 to 4, 8-wave
    workgroups) against the oracle: partial last blocks, an empty sequence,
    split ranges; and it is a different kernel from the matrix one (its
    rounding differs somewhere)."""
    import torch
    from tests import gpu_util as gu
    from workloads.configs import host_normal, deal_tables
    rng = np.random.default_rng(hq * 17 + hkv + d)
    lens = np.array([600, 1500, 2047, 900, 3000, 17, 0, 700], dtype=np.int64)
    need = int(sum(-(-x // 16) for x in lens))
    table = deal_tables(rng.permutation(need + 5)[:need].astype(np.int32), lens, 256)
    dp = gu.DevicePool(1, need + 5, hkv, d, dtype)
    fill_random_pool(dp, 31)
    q = host_normal(rng, (len(lens), hq, d), dtype)
    check_decode_all(dp, 0, q, table, lens, hq, parts=(0, 512), variants=("dot2",))
    q_dev = gu.to_device_raw(q.reshape(-1), dtype).view(q.shape)
    tdev = torch.from_numpy(table).cuda()
    os.environ["PKV_DECODE_KERNEL"] = "2"
    try:
        out2, _ = gu.decode(dp, 0, q_dev, tdev, lens, hq, 0)
    finally:
        os.environ.pop("PKV_DECODE_KERNEL", None)
    out0, _ = gu.decode(dp, 0, q_dev, tdev, lens, hq, 0)
    assert not torch.equal(out2, out0), "the packed-dot-product kernel did not run"


@pytest.mark.parametrize("dtype,hq,hkv,d", [("bf16", 32, 8, 128), ("f16", 64, 64, 128),
                                           ("bf16", 8, 8, 64), ("f16", 16, 4, 64)])
def test_lds_staged_variant(dtype, hq, hkv, d):
    """Attention alone with K and V staged through LDS by direct loads (kernel
    variant 12: one tile, 8-wave workgroups, two blocks in flight per wave)
    against the oracle, with partial last blocks, an empty sequence and split
    ranges; and bit for bit equal to the default kernel, which takes the same
    values in the same order from registers."""
    import torch
    from tests import gpu_util as gu
    from workloads.configs import host_normal, deal_tables
    rng = np.random.default_rng(hq * 13 + hkv + d)
    lens = np.array([600, 1500, 2047, 900, 3000, 17, 0, 700, 1024, 515], dtype=np.int64)
    need = int(sum(-(-x // 16) for x in lens))
    table = deal_tables(rng.permutation(need + 5)[:need].astype(np.int32), lens, 256)
    dp = gu.DevicePool(1, need + 5, hkv, d, dtype)
    fill_random_pool(dp, 37)
    q = host_normal(rng, (len(lens), hq, d), dtype)
    check_decode_all(dp, 0, q, table, lens, hq, parts=(0, 512), variants=("staged",))
    q_dev = gu.to_device_raw(q.reshape(-1), dtype).view(q.shape)
    tdev = torch.from_numpy(table).cuda()
    for part in (0, 512):
        os.environ["PKV_DECODE_KERNEL"] = "12"
        try:
            out12, lse12 = gu.decode(dp, 0, q_dev, tdev, lens, hq, part)
        finally:
            os.environ.pop("PKV_DECODE_KERNEL", None)
        out0, lse0 = gu.decode(dp, 0, q_dev, tdev, lens, hq, part)
        assert torch.equal(out12, out0) and torch.equal(lse12, lse0), "staged vs register path"


def test_launch_order_chunks_cover_every_item():
    """A launch of many rounds of workgroups per CU takes its items in chunks
    of 8 (each XCD takes whole items); with a partial last chunk every
    (item, KV head) is still served once: the result equals the oracle, and
    it is bit for bit the same in item-major order and in chunks of 3 and 5
    (the order changes no arithmetic)."""
    import torch
    from tests import gpu_util as gu
    from workloads.configs import host_normal, deal_tables
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    hkv, hq, d = 32, 32, 64
    n = -(-16 * cus // hkv) + 3          # at least 16 workgroups per CU, n % 8 != 0
    if n % 8 == 0:
        n += 1
    rng = np.random.default_rng(2024)
    lens = rng.integers(1, 200, size=n).astype(np.int64)
    lens[:4] = [0, 1, 16, 17]
    need = int(sum(-(-x // 16) for x in lens))
    table = deal_tables(rng.permutation(need + 3)[:need].astype(np.int32), lens, 16)
    dp = gu.DevicePool(1, need + 3, hkv, d, "f16")
    fill_random_pool(dp, 41)
    q = host_normal(rng, (n, hq, d), "f16")
    gu.say("launch order: %d sequences x %d KV heads on %d CUs" % (n, hkv, cus))
    check_decode_all(dp, 0, q, table, lens, hq)
    q_dev = gu.to_device_raw(q.reshape(-1), "f16").view(q.shape)
    tdev = torch.from_numpy(table).cuda()
    out8, lse8 = gu.decode(dp, 0, q_dev, tdev, lens, hq, 0)
    for chunk in ("1", "3", "5"):
        os.environ["PKV_DECODE_CHUNK"] = chunk
        try:
            out, lse = gu.decode(dp, 0, q_dev, tdev, lens, hq, 0)
        finally:
            os.environ.pop("PKV_DECODE_CHUNK", None)
        assert torch.equal(out, out8) and torch.equal(lse, lse8), "chunks of %s" % chunk


@pytest.mark.parametrize("n_seqs,inline", [(128, True), (129, False)])
def test_plan_in_kernel_arguments(n_seqs, inline):
    """Plans of at most 128 items with no split travel in the kernel
    arguments: their upload leaves the workspace untouched, and decode is
    still right; one item more goes through the workspace."""
    import torch
    import paged_kv_cache_inject_amd as pkv
    from oracle import attention as o_att
    from tests import gpu_util as gu
    from workloads.configs import host_normal, deal_tables
    rng = np.random.default_rng(n_seqs)
    hq, hkv, d, dtype = 8, 2, 64, "bf16"
    lens = rng.integers(0, 90, size=n_seqs).astype(np.int64)
    need = int(sum(-(-x // 16) for x in lens))
    nb = need + 5
    table = deal_tables(rng.permutation(nb)[:need].astype(np.int32), lens, 8)
    dp = gu.DevicePool(1, nb, hkv, d, dtype)
    fill_random_pool(dp, 23)
    q = host_normal(rng, (n_seqs, hq, d), dtype)
    plan = pkv.pkv_decode_plan_create(lens, hq, hkv, d, 128)
    try:
        assert pkv.pkv_decode_plan_items(plan) == n_seqs      # no sequence split
        n_ws = pkv.pkv_decode_workspace_bytes(plan)
        ws = torch.full((n_ws,), 0x5A, dtype=torch.uint8, device="cuda")
        pkv.pkv_decode_plan_upload(plan, ws)
        torch.cuda.synchronize()
        untouched = bool((ws == 0x5A).all())
        assert untouched == inline, (n_seqs, untouched)
        q_dev = gu.to_device_raw(q.reshape(-1), dtype).view(q.shape)
        tables_dev = torch.from_numpy(np.ascontiguousarray(table, dtype=np.int32)).cuda()
        out = torch.full((n_seqs, hq, d), float("nan"), device="cuda")
        lse = torch.full((n_seqs, hq), float("nan"), device="cuda")
        pkv.pkv_decode_attention(plan, dp.desc(), 0, q_dev, tables_dev, out, lse, ws)
        torch.cuda.synchronize()
    finally:
        pkv.pkv_decode_plan_destroy(plan)
    kp, vp = dp.oracle_arrays(dp.host_copy())
    ref, ref_lse = o_att.decode_paged(q, kp, vp, dp.spec(), 0, [list(r) for r in table], lens,
                                      hq, by_plane=True)
    gu.assert_close(out.cpu().numpy(), ref, "out")
    gu.assert_close(lse.cpu().numpy(), ref_lse, "lse")
