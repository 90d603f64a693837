"""Calls that have nothing to do, through the C ABI on the GPU: an inject
call with no runs, one whose runs are all empty, one over an empty layer
range; an append of no tokens and an append for no sequences; a decode step
(attention alone and with the fused append) over an empty batch.  Each
returns success, leaves the pool byte for byte as the oracle leaves it
(unchanged), and leaves the cache's lengths as the oracle has them.  [InferScale] §3 (the scatter write
through the slot mapping: an empty mapping writes nothing); [KV essay]
"The fix" (one decode step per token: a batch of no sequences has no step).
"""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def test_calls_with_nothing_to_do_touch_nothing():
    import torch
    import paged_kv_cache_inject_amd as pkv
    from oracle import inject as o_inject
    from oracle.allocator import AllocatorModel
    from oracle.rope import rope_table
    from tests import gpu_util as gu
    from workloads.configs import host_normal

    gu.say("zero-size calls: inject, append, decode")
    L, H, NB, d, max_pos, hq = 2, 2, 8, 64, 64, 4
    fill = 0x7FAB
    dp = gu.DevicePool(L, NB, H, d, "bf16", fill_bits=fill)
    ref = np.full(dp.total, fill, dtype=np.uint16)
    kp, vp = dp.oracle_arrays(ref)
    cache = pkv.pkv_cache_create(NB, 2, 16, free_list_seed=3)
    model = AllocatorModel(NB, 2, 16, seed=3)
    pkv.pkv_alloc_blocks(cache, 0, 40)
    model.alloc_blocks(0, 40)
    rng = np.random.default_rng(11)
    n_src = 8
    src_k = host_normal(rng, (L, n_src, H, d), "bf16")
    src_v = host_normal(rng, (L, n_src, H, d), "bf16")
    dk = gu.to_device_raw(src_k.reshape(-1), "bf16")
    dv = gu.to_device_raw(src_v.reshape(-1), "bf16")
    src = pkv.make_src(dk, dv, n_src * H * d, H * d, n_src)
    o_cos, o_sin = rope_table(d, 10000.0, max_pos)
    _, _, dcos, dsin = gu.rope_tables(d, max_pos)
    lens = [0, 0]

    # inject: no runs; only empty runs (two of them past the reserved blocks
    # and the rotary table); a run over an empty layer range
    empty_runs = [(0, 0, 0, 0), (0, 0, 5, 3), (0, 0, 200, 0), (1, 0, 90, 0)]
    for runs, lb, le in (([], 0, L), (empty_runs, 0, L), ([(0, 6, 0, 0)], 1, 1)):
        ws = gu.workspace(pkv.pkv_inject_workspace_bytes(runs))
        pkv.pkv_inject(cache, dp.desc(), src, runs, lb, le, "pairs", dcos, dsin, max_pos, ws)
        torch.cuda.synchronize()
        lens = o_inject.inject(kp, vp, dp.spec(), model.tables, lens, runs, src_k.reshape(-1),
                               src_v.reshape(-1), n_src * H * d, H * d, lb, le, "pairs", o_cos,
                               o_sin)
        gu.assert_bytes_equal(dp.host_copy(), ref,
                              "pool after inject %r on [%d, %d)" % (runs, lb, le))
    _, glens = pkv.pkv_block_table(cache, range(2), 16)
    assert list(glens) == list(lens)
    assert np.array_equal(ref, np.full(dp.total, fill, dtype=np.uint16)), \
        "the oracle wrote something for a call with nothing to write"

    # append: no tokens for one sequence; no sequences
    tables, _ = pkv.pkv_block_table(cache, [0], 16)
    dtab = torch.from_numpy(np.ascontiguousarray(tables)).cuda()
    first = torch.tensor([3], dtype=torch.int32, device="cuda")
    kn = torch.zeros(H * d, dtype=torch.bfloat16, device="cuda")
    vn = torch.zeros(H * d, dtype=torch.bfloat16, device="cuda")
    pkv.pkv_append_kv(dp.desc(), 0, dtab, first, 0, kn, vn, "pairs", dcos, dsin, max_pos)
    pkv.pkv_append_kv(dp.desc(), 1, dtab[:0], first[:0], 1, kn, vn, "pairs", dcos, dsin, max_pos)
    torch.cuda.synchronize()
    gu.assert_bytes_equal(dp.host_copy(), ref, "pool after appends of nothing")

    # decode over an empty batch, attention alone and with the fused append
    plan = pkv.pkv_decode_plan_create(np.zeros(0, dtype=np.int64), hq, H, d)
    try:
        ws = gu.workspace(pkv.pkv_decode_workspace_bytes(plan))
        pkv.pkv_decode_plan_upload(plan, ws)
        q = torch.zeros(0, hq, d, dtype=torch.bfloat16, device="cuda")
        out = torch.zeros(0, hq, d, device="cuda")
        lse = torch.zeros(0, hq, device="cuda")
        empty_tab = torch.zeros(0, 4, dtype=torch.int32, device="cuda")
        pkv.pkv_decode_attention(plan, dp.desc(), 0, q, empty_tab, out, lse, ws)
        knew = torch.zeros(0, H, d, dtype=torch.bfloat16, device="cuda")
        pkv.pkv_append_decode_attention(plan, dp.desc(), 1, q, empty_tab, knew, knew, "pairs",
                                        dcos, dsin, max_pos, out, lse, ws)
        torch.cuda.synchronize()
    finally:
        pkv.pkv_decode_plan_destroy(plan)
    gu.assert_bytes_equal(dp.host_copy(), ref, "pool after decode over an empty batch")
    pkv.pkv_cache_destroy(cache)
