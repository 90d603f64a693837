"""Tiny fp32 reference workload, end to end through the C ABI, against the
oracle: prefill by inject, a 24-token unrotated chunk injected over
positions 40..63 of sequence 1, then decode (several split sizes)."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def run_tiny(part_tokens_list=(0, 16, 32, 48)):
    import torch
    import paged_kv_cache_inject_amd as pkv
    from oracle import inject as o_inject, attention as o_att
    from oracle.allocator import AllocatorModel
    from oracle.rope import rope_table
    from tests import gpu_util as gu
    from workloads.configs import TINY, tiny_inputs

    cfg = TINY
    w = tiny_inputs(cfg)
    L, H, d = cfg.n_layers, cfg.n_kv_heads, cfg.head_dim
    max_pos = 128
    dp = gu.DevicePool(L, w["num_blocks"], H, d, "f32", fill_bits=0x7FC0DEAD)
    cos, sin, dcos, dsin = gu.rope_tables(d, max_pos)

    # library allocator with the workload's tables
    cache = pkv.pkv_cache_create(w["num_blocks"], 2, w["max_blocks"])
    model = AllocatorModel(w["num_blocks"], 2, w["max_blocks"])
    for s in range(2):
        ids = [b for b in w["tables"][s] if b >= 0]
        pkv.pkv_set_blocks(cache, s, ids, 0)
        model.set_blocks(s, ids, 0)

    src_k = gu.to_device_raw(w["src_k"].reshape(-1), "f32")
    src_v = gu.to_device_raw(w["src_v"].reshape(-1), "f32")
    n_src = w["src_k"].shape[1]
    src = pkv.make_src(src_k, src_v, n_src * H * d, H * d, n_src)
    for runs in (w["prefill_runs"], w["chunk_runs"]):
        ws = gu.workspace(pkv.pkv_inject_workspace_bytes(runs))
        pkv.pkv_inject(cache, dp.desc(), src, runs, 0, L, "pairs", dcos, dsin, max_pos, ws)
        torch.cuda.synchronize()

    # oracle
    ref = np.full(dp.total, np.uint32(0x7FC0DEAD).view(np.float32), dtype=np.float32)
    kp, vp = dp.oracle_arrays(ref)
    o_cos, o_sin = rope_table(d, cfg.rope_base, max_pos)
    lens = [0, 0]
    for runs in (w["prefill_runs"], w["chunk_runs"]):
        lens = o_inject.inject(kp, vp, dp.spec(), model.tables, lens, runs,
                               w["src_k"].reshape(-1), w["src_v"].reshape(-1), n_src * H * d,
                               H * d, 0, L, "pairs", o_cos, o_sin)
    got = dp.host_copy()
    gu.assert_bytes_equal(got, ref, "tiny pool after inject")

    table, glens = pkv.pkv_block_table(cache, [0, 1], w["max_blocks"])
    assert list(glens) == list(lens) == list(w["lens"])
    assert np.array_equal(table, w["tables"])

    q_dev = gu.to_device_raw(w["q"].reshape(-1), "f32").view(2, cfg.n_q_heads, d)
    tables_dev = torch.from_numpy(table).cuda()
    ref_out, ref_lse = o_att.decode_paged(w["q"], kp, vp, dp.spec(), 0, model.tables, lens,
                                          cfg.n_q_heads)
    for part in part_tokens_list:
        out, lse = gu.decode(dp, 0, q_dev, tables_dev, lens, cfg.n_q_heads, part)
        gu.assert_close(out.cpu().numpy(), ref_out, "tiny out part=%d" % part)
        gu.assert_close(lse.cpu().numpy(), ref_lse, "tiny lse part=%d" % part)
    pkv.pkv_cache_destroy(cache)


def test_tiny_reference_workload():
    run_tiny()
