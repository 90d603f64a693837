"""The decode step as the benchmark times it: pkv_append_decode_attention on
sequences long enough that the planner gives each (token range, KV head)
workgroup 8 waves, which is the kernel instance (8 waves, fused append of the
step's own token, one workgroup per CU on uniform batches) behind the
headline figure.  [KV essay] "The fix": each step appends its token's K/V
entry and attends over the cache including it; [InferScale] §2: the key is
stored rotated to its own position.

Every case checks, on the same seeded inputs:
* the planner chose 8 waves for the plan (pkv_decode_plan_waves);
* the pool blocks the step writes, out and lse are byte for byte those of
  the two-call path (pkv_append_kv at len - 1, then pkv_decode_attention);
* the written planes equal the oracle's append exactly, and out/lse match
  the oracle's decode within 1e-3 + 2e-3 |ref| (all sequences, or a sample at
  the full 70B and ragged sizes).
Shapes: the Llama-3-70B-shaped 80-layer workload at full size (layers 0, 41
and 79), the Llama-3-8B-shaped layer in full, the ragged MHA batch (sampled),
fp8 pools with per-head and per-block scales on long sequences, two tiles of
16 query heads (G = 32), four tiles (G = 64), d = 64, the halves pairing and
a sliding window.
"""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def _fill_normal(dp, seed):
    from workloads.configs import device_normal
    for layer in range(dp.n_layers):
        a, b = layer * dp.layer_stride, (layer + 1) * dp.layer_stride
        dp.buf[a:b] = device_normal(b - a, dp.dtype, seed * 1000 + layer)


def _fill_fp8(dp, rng):
    """Random finite E4M3 codes of either sign (no NaN code)."""
    import torch
    codes = rng.integers(0, 0x70, size=dp.total, dtype=np.uint8)
    codes |= (rng.integers(0, 2, size=dp.total, dtype=np.uint8) << 7).astype(np.uint8)
    dp.buf.copy_(torch.from_numpy(codes))


def _bits(t):
    import torch
    return t.view(torch.uint8) if t.dtype == torch.uint8 else t.view(torch.int16)


def run_step(dp, layer, lens, hq, q_dev, tdev, kd, vd, mode, qdt, max_pos, seqs, q_host,
             k_host, v_host, table, part=0, window=0, ks=None, vs=None, want_waves=8):
    """One decode step of `layer` through the one-launch call, checked against
    the two-call path and the oracle.  `seqs`: sequences compared with the
    oracle (all when None)."""
    import torch
    import paged_kv_cache_inject_amd as pkv
    from oracle import attention as o_att, inject as o_inject
    from oracle.rope import rope_table
    from tests import gpu_util as gu

    B = len(lens)
    hkv, d = dp.n_kv_heads, dp.head_dim
    live = [b for b in range(B) if lens[b] > 0]
    sel = live if seqs is None else [b for b in seqs if lens[b] > 0]
    # the blocks the step writes: the one holding position len - 1 of each sequence
    touched = sorted({int(table[b][(int(lens[b]) - 1) // 16]) for b in live})
    idx = torch.tensor(touched, dtype=torch.long, device="cuda")
    view = dp.buf[layer * dp.layer_stride:(layer + 1) * dp.layer_stride].view(
        dp.num_blocks, dp.block_stride)
    saved = view.index_select(0, idx).clone()
    before = gu.host_planes_for(dp, layer, table, sel, None)      # oracle input

    plan = pkv.pkv_decode_plan_create(lens, hq, hkv, d, part, window=window)
    try:
        waves = pkv.pkv_decode_plan_waves(plan)
        assert waves == want_waves, "planner chose %d waves" % waves
        ws = gu.workspace(pkv.pkv_decode_workspace_bytes(plan))
        pkv.pkv_decode_plan_upload(plan, ws)
        out1 = torch.full((B, hq, d), float("nan"), device="cuda")
        lse1 = torch.full((B, hq), float("nan"), device="cuda")
        gu.say("  one-launch step: layer", layer, "items", pkv.pkv_decode_plan_items(plan),
               "part", pkv.pkv_decode_plan_part_tokens(plan), "waves", waves)
        pkv.pkv_append_decode_attention(plan, dp.desc(), layer, q_dev, tdev, kd, vd, mode, dcos_of(dp),
                                        dsin_of(dp), max_pos, out1, lse1, ws, q_dtype=qdt)
        torch.cuda.synchronize()
        after1 = view.index_select(0, idx).clone()
        # the same step as two calls, from the saved blocks
        view.index_copy_(0, idx, saved)
        first = torch.from_numpy((np.asarray(lens) - 1).astype(np.int32)).cuda()
        pkv.pkv_append_kv(dp.desc(), layer, tdev, first, 1, kd, vd, mode, dcos_of(dp),
                          dsin_of(dp), max_pos, new_dtype=qdt)
        out2 = torch.full((B, hq, d), float("nan"), device="cuda")
        lse2 = torch.full((B, hq), float("nan"), device="cuda")
        pkv.pkv_decode_attention(plan, dp.desc(), layer, q_dev, tdev, out2, lse2, ws, q_dtype=qdt)
        torch.cuda.synchronize()
    finally:
        pkv.pkv_decode_plan_destroy(plan)
    after2 = view.index_select(0, idx)
    assert torch.equal(_bits(after1), _bits(after2)), "written blocks: one call vs two calls"
    assert torch.equal(out1, out2), "out: one call vs two calls"
    assert torch.equal(lse1, lse2), "lse: one call vs two calls"

    # oracle: append the newest token, then decode
    o_cos, o_sin = rope_table(d, 10000.0, max_pos)
    kp, vp = dp.oracle_arrays(before)
    rows = [list(r) for r in table]
    o_inject.append(kp, vp, dp.spec(), layer, rows, lens, sel, 1, k_host[sel][:, None],
                    v_host[sel][:, None], mode, o_cos, o_sin, src_dtype=qdt, k_scale=ks,
                    v_scale=vs)
    got = gu.host_planes_for(dp, layer, table, sel, None)
    gu.assert_bytes_equal(got, before, "pool vs oracle append")
    ref, ref_lse = o_att.decode_paged(q_host, kp, vp, dp.spec(), layer, rows, lens, hq, seqs=sel,
                                      by_plane=True, q_dtype=qdt, k_scale=ks, v_scale=vs,
                                      window=window or None)
    o, ls = out1.cpu().numpy(), lse1.cpu().numpy()
    worst = gu.assert_close(o[sel], ref[sel], "out vs oracle")
    gu.assert_close(ls[sel], ref_lse[sel], "lse vs oracle")
    gu.say("  layer", layer, "sequences checked", len(sel), "worst abs err %.3g" % worst)
    return worst


# rotary tables live on the pool object for the duration of a test
def dcos_of(dp):
    return dp.rope[0]


def dsin_of(dp):
    return dp.rope[1]


def _attach_rope(dp, max_pos):
    from tests import gpu_util as gu
    _, _, dcos, dsin = gu.rope_tables(dp.head_dim, max_pos)
    dp.rope = (dcos, dsin)


def _new_rows(rng, B, hkv, d, qdt):
    from tests import gpu_util as gu
    from workloads.configs import host_normal
    k = host_normal(rng, (B, hkv, d), qdt)
    v = host_normal(rng, (B, hkv, d), qdt)
    return k, v, gu.to_device_raw(k.reshape(-1), qdt), gu.to_device_raw(v.reshape(-1), qdt)


def test_llama70b_step_full_size_layers_0_41_79():
    """The benchmark's workload itself: 80 layers x 16,384 blocks (85.9 GB),
    32 sequences of 8,192 tokens under the shuffled table, 64 query / 8 KV
    heads; one plan for the step, three layers run and checked, three
    sequences per layer against the oracle and all 32 against the two-call
    path."""
    import torch
    from tests import gpu_util as gu
    from workloads.configs import LLAMA70B_80LAYER, llama70b_structure, host_normal
    cfg = LLAMA70B_80LAYER
    st = llama70b_structure(cfg)
    gu.say("70B step: 80 layers x", st["num_blocks"], "blocks")
    dp = gu.DevicePool(cfg.n_layers, st["num_blocks"], cfg.n_kv_heads, cfg.head_dim, cfg.dtype)
    _fill_normal(dp, cfg.seed)
    lens = st["lens"]
    max_pos = int(lens.max())
    _attach_rope(dp, max_pos)
    q = host_normal(st["rng"], (cfg.batch, cfg.n_q_heads, cfg.head_dim), cfg.dtype)
    q_dev = gu.to_device_raw(q.reshape(-1), cfg.dtype).view(q.shape)
    tdev = torch.from_numpy(st["tables"]).cuda()
    rng = np.random.default_rng(703)
    for layer in (0, 41, 79):
        k, v, kd, vd = _new_rows(rng, cfg.batch, cfg.n_kv_heads, cfg.head_dim, cfg.dtype)
        seqs = sorted(np.random.default_rng(layer).choice(cfg.batch, 3, replace=False).tolist())
        run_step(dp, layer, lens, cfg.n_q_heads, q_dev, tdev, kd, vd, "pairs", cfg.dtype,
                 max_pos, seqs, q, k, v, st["tables"])
    del dp
    torch.cuda.empty_cache()


def test_llama8b_step_full():
    """The Llama-3-8B-shaped layer (64 sequences, lengths 512..4096): every
    sequence against the oracle."""
    import torch
    from tests import gpu_util as gu
    from workloads.configs import LLAMA8B_1LAYER, llama8b_structure, host_normal
    cfg = LLAMA8B_1LAYER
    st = llama8b_structure(cfg)
    gu.say("8B step: pool", st["num_blocks"], "blocks")
    dp = gu.DevicePool(1, st["num_blocks"], cfg.n_kv_heads, cfg.head_dim, cfg.dtype)
    _fill_normal(dp, cfg.seed)
    lens = st["lens"]
    max_pos = int(lens.max())
    _attach_rope(dp, max_pos)
    q = host_normal(st["rng"], (cfg.batch, cfg.n_q_heads, cfg.head_dim), cfg.dtype)
    q_dev = gu.to_device_raw(q.reshape(-1), cfg.dtype).view(q.shape)
    tdev = torch.from_numpy(st["tables"]).cuda()
    k, v, kd, vd = _new_rows(np.random.default_rng(802), cfg.batch, cfg.n_kv_heads,
                             cfg.head_dim, cfg.dtype)
    run_step(dp, 0, lens, cfg.n_q_heads, q_dev, tdev, kd, vd, "pairs", cfg.dtype, max_pos, None,
             q, k, v, st["tables"])


def test_many_workgroups_step_appends_in_its_own_launch():
    """A launch of at least 16 workgroups per CU (128 sequences x 32 KV heads
    of 520..700 tokens, f16 and bf16, one sequence empty): the step appends in
    a launch of its own and then runs attention alone.  Pool, out and lse
    byte for byte those of the two calls; every live sequence against the
    oracle; the empty sequence gets no write."""
    import torch
    from tests import gpu_util as gu
    from workloads.configs import deal_tables, host_normal
    for dtype, seed in (("f16", 31), ("bf16", 32)):
        rng = np.random.default_rng(seed)
        B, hkv, hq, d = 128, 32, 32, 128
        lens = rng.integers(520, 700, size=B).astype(np.int64)
        lens[7] = 0
        need = int(sum(-(-int(x) // 16) for x in lens))
        nb = need + 8
        table = deal_tables(rng.permutation(nb)[:need].astype(np.int32), lens, 64)
        gu.say("many-workgroup step", dtype, "pool", nb, "blocks")
        dp = gu.DevicePool(1, nb, hkv, d, dtype)
        _fill_normal(dp, seed)
        max_pos = int(lens.max())
        _attach_rope(dp, max_pos)
        q = host_normal(rng, (B, hq, d), dtype)
        q_dev = gu.to_device_raw(q.reshape(-1), dtype).view(q.shape)
        tdev = torch.from_numpy(table).cuda()
        k, v, kd, vd = _new_rows(rng, B, hkv, d, dtype)
        run_step(dp, 0, lens, hq, q_dev, tdev, kd, vd, "pairs", dtype, max_pos, None, q, k, v,
                 table)
        del dp
        torch.cuda.empty_cache()


@pytest.mark.parametrize("blockwise", [False, True])
def test_many_workgroups_fp8_step_in_one_launch(blockwise):
    """fp8 pools keep the one-launch step on launches of many rounds of
    workgroups per CU: the items are taken in chunks of 8 (here with a
    partial last chunk) and two of the fused instance's workgroups share a
    CU.  131+ sequences x 32 KV heads of 520..700 tokens, scales per head or
    per block, one sequence empty: pool, out and lse byte for byte those of
    the two calls; every live sequence against the oracle."""
    import torch
    from tests import gpu_util as gu
    from workloads.configs import deal_tables, host_normal
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    hkv, hq, d = 32, 32, 128
    B = -(-16 * cus // hkv) + 3           # at least 16 workgroups per CU, B % 8 != 0
    if B % 8 == 0:
        B += 1
    rng = np.random.default_rng(77 + blockwise)
    lens = rng.integers(520, 700, size=B).astype(np.int64)
    lens[5] = 0
    need = int(sum(-(-int(x) // 16) for x in lens))
    nb = need + 8
    table = deal_tables(rng.permutation(nb)[:need].astype(np.int32), lens, 64)
    gu.say("many-workgroup fp8 step: %d sequences, pool %d blocks, per-block scales %s"
           % (B, nb, blockwise))
    dp = gu.DevicePool(1, nb, hkv, d, "fp8")
    shape = (1, nb, hkv) if blockwise else (1, hkv)
    ks = rng.uniform(0.01, 0.03, size=shape).astype(np.float32)
    vs = rng.uniform(0.01, 0.03, size=shape).astype(np.float32)
    dp.set_scales(ks, vs)
    _fill_fp8(dp, rng)
    max_pos = int(lens.max())
    _attach_rope(dp, max_pos)
    q = host_normal(rng, (B, hq, d), "bf16")
    q_dev = gu.to_device_raw(q.reshape(-1), "bf16").view(q.shape)
    tdev = torch.from_numpy(table).cuda()
    k, v, kd, vd = _new_rows(rng, B, hkv, d, "bf16")
    run_step(dp, 0, lens, hq, q_dev, tdev, kd, vd, "pairs", "bf16", max_pos, None, q, k, v,
             table, ks=ks, vs=vs)
    del dp
    torch.cuda.empty_cache()


def test_ragged_mha_step_sampled():
    """The ragged MHA batch (256 sequences, lognormal lengths, 64 KV heads,
    f16): 24 sequences (shortest, longest, random) against the oracle, all of
    them against the two-call path."""
    import torch
    from tests import gpu_util as gu
    from workloads.configs import RAGGED_MHA, ragged_mha_structure, host_normal
    cfg = RAGGED_MHA
    st = ragged_mha_structure(cfg)
    lens = st["lens"]
    gu.say("ragged MHA step: pool", st["num_blocks"], "blocks, max len", int(lens.max()))
    dp = gu.DevicePool(1, st["num_blocks"], cfg.n_kv_heads, cfg.head_dim, cfg.dtype)
    _fill_normal(dp, cfg.seed)
    max_pos = int(lens.max())
    _attach_rope(dp, max_pos)
    q = host_normal(st["rng"], (cfg.batch, cfg.n_q_heads, cfg.head_dim), cfg.dtype)
    q_dev = gu.to_device_raw(q.reshape(-1), cfg.dtype).view(q.shape)
    tdev = torch.from_numpy(st["tables"]).cuda()
    k, v, kd, vd = _new_rows(np.random.default_rng(905), cfg.batch, cfg.n_kv_heads,
                             cfg.head_dim, cfg.dtype)
    order = np.argsort(lens)
    seqs = sorted(set(order[:6].tolist() + order[-6:].tolist() +
                      np.random.default_rng(1).choice(cfg.batch, 12, replace=False).tolist()))
    run_step(dp, 0, lens, cfg.n_q_heads, q_dev, tdev, kd, vd, "halves", cfg.dtype, max_pos, seqs,
             q, k, v, st["tables"])
    del dp
    torch.cuda.empty_cache()


LONG = np.array([8192, 4000, 600, 8192, 3001, 1200, 7777, 2048], dtype=np.int64)

CASES = [
    # pool, query heads, KV heads, head dim, pairing, part tokens, window
    ("fp8", 64, 8, 128, "pairs", 0, 0),         # per-(layer, head) scales
    ("fp8b", 64, 8, 128, "pairs", 0, 0),        # per-(layer, block, head) scales
    ("fp8", 32, 8, 64, "halves", 0, 0),
    ("bf16", 64, 2, 128, "pairs", 0, 0),        # G = 32: two tiles of 16 query heads
    ("f16", 64, 1, 128, "halves", 0, 0),        # G = 64: four tiles (4-wave workgroups)
    ("bf16", 64, 8, 64, "pairs", 0, 0),         # d = 64
    ("bf16", 32, 8, 128, "halves", 1024, 0),    # split ranges merged afterwards
    ("bf16", 32, 8, 128, "pairs", 0, 1500),     # sliding window
]


@pytest.mark.parametrize("dtype,hq,hkv,d,mode,part,window", CASES)
def test_long_sequences_step(dtype, hq, hkv, d, mode, part, window):
    import torch
    from tests import gpu_util as gu
    from workloads.configs import host_normal, deal_tables
    gu.say("8-wave step", dtype, hq, hkv, d, mode, part, window)
    blockwise = dtype == "fp8b"
    dtype = "fp8" if blockwise else dtype
    rng = np.random.default_rng(hq * 1013 + hkv * 37 + d + part + window + blockwise)
    L, layer = 2, 1
    lens = LONG.copy()
    need = int(sum(-(-int(x) // 16) for x in lens))
    nb = need + 9
    table = deal_tables(rng.permutation(nb)[:need].astype(np.int32), lens, 512)
    dp = gu.DevicePool(L, nb, hkv, d, dtype)
    ks = vs = None
    if dtype == "fp8":
        shape = (L, nb, hkv) if blockwise else (L, hkv)
        ks = rng.uniform(0.01, 0.03, size=shape).astype(np.float32)
        vs = rng.uniform(0.01, 0.03, size=shape).astype(np.float32)
        dp.set_scales(ks, vs)
        _fill_fp8(dp, rng)
    else:
        _fill_normal(dp, 41 + hkv)
    qdt = "bf16" if dtype == "fp8" else dtype
    max_pos = int(lens.max())
    _attach_rope(dp, max_pos)
    q = host_normal(rng, (len(lens), hq, d), qdt)
    q_dev = gu.to_device_raw(q.reshape(-1), qdt).view(q.shape)
    tdev = torch.from_numpy(table).cuda()
    k, v, kd, vd = _new_rows(rng, len(lens), hkv, d, qdt)
    run_step(dp, layer, lens, hq, q_dev, tdev, kd, vd, mode, qdt, max_pos, None, q, k, v, table,
             part=part, window=window, ks=ks, vs=vs)
