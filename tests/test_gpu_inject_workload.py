"""The injection workload end to end through the C ABI: top-8 retrieved
chunks composed per request at non-consecutive positions (after a fixed
32-token prefix, each chunk behind a gap filled from a separator), one
inject call over all 32 layers, a 32-token suffix and one decode token
appended, then decode over every layer.  Layers 0 and 31 are checked
against the oracle: the pool byte for byte, the attention outputs within
tolerance.  Run at a reduced store size and at the full 10,000-chunk size
(the configuration the benchmark times)."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def run_inject_workload(n_chunks, batch=None, check_layers=(0, 31), decode_seqs=None):
    import torch
    import paged_kv_cache_inject_amd as pkv
    from oracle import attention as o_att, inject as o_inject
    from oracle.allocator import AllocatorModel
    from oracle.layout import PoolSpec
    from oracle.rope import rope_table
    from tests import gpu_util as gu
    from workloads.configs import INJECT_TOP8, inject_structure, device_normal, host_normal

    cfg = INJECT_TOP8
    st = inject_structure(cfg, n_chunks=n_chunks, batch=batch)
    L, H, d, HQ = cfg.n_layers, cfg.n_kv_heads, cfg.head_dim, cfg.n_q_heads
    B = len(st["mem_lens"])
    row = H * d
    n_src = st["n_src"]
    suffix = cfg.extra["suffix"]
    gu.say("inject workload: %d chunks, %d source tokens, %d runs, pool %d blocks"
           % (n_chunks, n_src, len(st["runs"]), st["num_blocks"]))
    store_k = torch.empty(L * n_src * row, dtype=torch.bfloat16, device="cuda")
    store_v = torch.empty(L * n_src * row, dtype=torch.bfloat16, device="cuda")
    for layer in range(L):
        a, b = layer * n_src * row, (layer + 1) * n_src * row
        store_k[a:b] = device_normal(b - a, "bf16", cfg.seed * 1000 + 2 * layer)
        store_v[a:b] = device_normal(b - a, "bf16", cfg.seed * 1000 + 2 * layer + 1)
    dp = gu.DevicePool(L, st["num_blocks"], H, d, "bf16", fill_bits=0x7FAB)

    cache = pkv.pkv_cache_create(st["num_blocks"], B, st["max_blocks"], st["free_list_seed"])
    model = AllocatorModel(st["num_blocks"], B, st["max_blocks"], seed=st["free_list_seed"])
    for b_, m in enumerate(st["mem_lens"]):
        pkv.pkv_alloc_blocks(cache, b_, int(m))
        model.alloc_blocks(b_, int(m))
    max_pos = 4096
    cos, sin, dcos, dsin = gu.rope_tables(d, max_pos)
    o_cos, o_sin = rope_table(d, cfg.rope_base, max_pos)
    assert np.array_equal(cos, o_cos) and np.array_equal(sin, o_sin)
    src = pkv.make_src(store_k, store_v, n_src * row, row, n_src)
    runs = st["runs"]
    ws = gu.workspace(pkv.pkv_inject_workspace_bytes(runs))
    pkv.pkv_inject(cache, dp.desc(), src, runs, 0, L, "pairs", dcos, dsin, max_pos, ws)

    seqs = list(range(B))
    lens_after_inject = [int(x) for x in st["mem_lens"]]
    first_suffix = pkv.pkv_extend(cache, seqs, suffix)
    first_tok = pkv.pkv_extend(cache, seqs, 1)
    table, lens = pkv.pkv_block_table(cache, seqs, st["max_blocks"])
    for s_, n_ in enumerate(lens_after_inject):
        model.set_len(s_, n_)
    assert list(first_suffix) == model.extend(seqs, suffix)
    assert list(first_tok) == model.extend(seqs, 1)
    assert [list(r[r >= 0]) for r in table] == model.tables
    assert list(lens) == model.lens
    tdev = torch.from_numpy(table).cuda()
    f1 = torch.from_numpy(first_suffix.astype(np.int32)).cuda()
    f2 = torch.from_numpy(first_tok.astype(np.int32)).cuda()
    new_k, new_v = {}, {}
    for layer in range(L):
        ks = device_normal(B * suffix * row, "bf16", cfg.seed * 7000 + layer)
        vs = device_normal(B * suffix * row, "bf16", cfg.seed * 7000 + 100 + layer)
        kt = device_normal(B * row, "bf16", cfg.seed * 9000 + layer)
        vt = device_normal(B * row, "bf16", cfg.seed * 9000 + 100 + layer)
        pkv.pkv_append_kv(dp.desc(), layer, tdev, f1, suffix, ks, vs, "pairs", dcos, dsin, max_pos)
        pkv.pkv_append_kv(dp.desc(), layer, tdev, f2, 1, kt, vt, "pairs", dcos, dsin, max_pos)
        if layer in check_layers:
            new_k[layer] = (gu.raw_view(ks.cpu()).reshape(B, suffix, H, d),
                            gu.raw_view(kt.cpu()).reshape(B, 1, H, d))
            new_v[layer] = (gu.raw_view(vs.cpu()).reshape(B, suffix, H, d),
                            gu.raw_view(vt.cpu()).reshape(B, 1, H, d))
    q = host_normal(np.random.default_rng(cfg.seed + 1), (B, HQ, d), "bf16")
    q_dev = gu.to_device_raw(q.reshape(-1), "bf16").view(B, HQ, d)
    plan = pkv.pkv_decode_plan_create(lens, HQ, H, d, 0)
    dws = gu.workspace(pkv.pkv_decode_workspace_bytes(plan))
    pkv.pkv_decode_plan_upload(plan, dws)
    outs = {}
    for layer in range(L):
        out = torch.empty(B, HQ, d, device="cuda")
        lse = torch.empty(B, HQ, device="cuda")
        pkv.pkv_decode_attention(plan, dp.desc(), layer, q_dev, tdev, out, lse, dws)
        if layer in check_layers:
            outs[layer] = (out, lse)
    torch.cuda.synchronize()
    pkv.pkv_decode_plan_destroy(plan)

    # Oracle, one layer at a time, on a compact copy of the referenced source rows.
    used = np.unique(np.concatenate([np.arange(s_, s_ + n, dtype=np.int64)
                                     for (_, n, _, s_) in runs]))
    remap = {int(t): i for i, t in enumerate(used)}
    compact_runs = [(q_, n, p_, remap[s_]) for (q_, n, p_, s_) in runs]
    idx = torch.from_numpy(used).cuda()
    spec1 = PoolSpec(1, dp.num_blocks, H, d, "bf16", dp.layer_stride, dp.block_stride,
                     dp.head_stride)
    for layer in check_layers:
        gu.say("oracle layer", layer)
        base = layer * n_src * row
        sk = gu.raw_view(store_k[base:base + n_src * row].view(n_src, row).index_select(0, idx).cpu())
        sv = gu.raw_view(store_v[base:base + n_src * row].view(n_src, row).index_select(0, idx).cpu())
        ref = np.full(dp.layer_stride, 0x7FAB, dtype=np.uint16)
        kp, vp = ref, ref[dp.v_off:]
        o_lens = o_inject.inject(kp, vp, spec1, model.tables, [0] * B, compact_runs, sk.reshape(-1),
                                 sv.reshape(-1), 0, row, 0, 1, "pairs", o_cos, o_sin)
        assert o_lens == lens_after_inject
        lens_mid = [n_ + suffix for n_ in o_lens]
        o_inject.append(kp, vp, spec1, 0, model.tables, lens_mid, seqs, suffix,
                        new_k[layer][0], new_v[layer][0], "pairs", o_cos, o_sin)
        o_inject.append(kp, vp, spec1, 0, model.tables, model.lens, seqs, 1,
                        new_k[layer][1], new_v[layer][1], "pairs", o_cos, o_sin)
        got = gu.raw_view(dp.buf[layer * dp.layer_stride:(layer + 1) * dp.layer_stride].cpu())
        gu.assert_bytes_equal(got, ref, "pool layer %d after inject + append" % layer)
        chk = seqs if decode_seqs is None else decode_seqs
        r_out, r_lse = o_att.decode_paged(q, kp, vp, spec1, 0, model.tables, model.lens, HQ,
                                          seqs=chk, by_plane=True)
        o, l = outs[layer][0].cpu().numpy(), outs[layer][1].cpu().numpy()
        gu.assert_close(o[chk], r_out[chk], "decode out layer %d" % layer)
        gu.assert_close(l[chk], r_lse[chk], "decode lse layer %d" % layer)
    pkv.pkv_cache_destroy(cache)
    del store_k, store_v, dp
    torch.cuda.empty_cache()


def test_inject_workload_reduced_store():
    run_inject_workload(300, batch=16)


def test_inject_workload_full_size_sampled():
    run_inject_workload(10000, decode_seqs=[0, 9, 17, 33, 42, 63])
