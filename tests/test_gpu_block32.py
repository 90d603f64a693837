"""32-token blocks on the GPU ([Inside engines] "PagedAttention": blocks of
e.g. 16 or 32 tokens): a 32-token block is the pair of 16-token planes 2b,
2b+1, so the kernels read the same plane table.  The injection workload's
structure injected into a 32-token cache matches the oracle byte for byte,
and decodes bit-identically to the same tokens injected into a 16-token
cache (the arithmetic never sees physical ids)."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def test_inject_and_decode_with_32_token_blocks():
    import torch
    import paged_kv_cache_inject_amd as pkv
    from oracle import attention as o_att, inject as o_inject
    from oracle.allocator import AllocatorModel, expand_table
    from oracle.rope import rope_table
    from tests import gpu_util as gu
    from workloads.configs import INJECT_TOP8, inject_structure, host_normal

    cfg = INJECT_TOP8
    st = inject_structure(cfg, n_chunks=40, batch=6)
    L, H, d, HQ = 2, cfg.n_kv_heads, cfg.head_dim, cfg.n_q_heads
    n_src, row = st["n_src"], H * d
    rng = np.random.default_rng(32)
    src_k = host_normal(rng, (L, n_src, H, d), "bf16")
    src_v = host_normal(rng, (L, n_src, H, d), "bf16")
    dk = gu.to_device_raw(src_k.reshape(-1), "bf16")
    dv = gu.to_device_raw(src_v.reshape(-1), "bf16")
    src = pkv.make_src(dk, dv, n_src * row, row, n_src, dtype="bf16")
    max_pos = 4096
    o_cos, o_sin = rope_table(d, 10000.0, max_pos)
    _, _, dcos, dsin = gu.rope_tables(d, max_pos)
    B = len(st["mem_lens"])
    q = host_normal(rng, (B, HQ, d), "bf16")
    q_dev = gu.to_device_raw(q.reshape(-1), "bf16").view(B, HQ, d)
    outs = {}
    for bt in (16, 32):
        gu.say("block size", bt)
        nb = -(-st["num_blocks"] * 16 // bt) + 2             # cache blocks
        max_blocks = -(-st["max_blocks"] * 16 // bt) + 1
        dp = gu.DevicePool(L, nb * bt // 16, H, d, "bf16", fill_bits=0x7FAB)
        cache = pkv.pkv_cache_create(nb, B, max_blocks, st["free_list_seed"], block_tokens=bt)
        model = AllocatorModel(nb, B, max_blocks, seed=st["free_list_seed"], block_tokens=bt)
        for b_, m in enumerate(st["mem_lens"]):
            pkv.pkv_alloc_blocks(cache, b_, int(m))
            model.alloc_blocks(b_, int(m))
        ws = gu.workspace(pkv.pkv_inject_workspace_bytes(st["runs"]))
        pkv.pkv_inject(cache, dp.desc(), src, st["runs"], 0, L, "pairs", dcos, dsin, max_pos, ws)
        torch.cuda.synchronize()
        ref = np.full(dp.total, 0x7FAB, dtype=np.uint16)
        kp, vp = dp.oracle_arrays(ref)
        planes = [expand_table(t, bt) for t in model.tables]
        lens = o_inject.inject(kp, vp, dp.spec(), planes, [0] * B, st["runs"], src_k.reshape(-1),
                               src_v.reshape(-1), n_src * row, row, 0, L, "pairs", o_cos, o_sin)
        gu.assert_bytes_equal(dp.host_copy(), ref, "pool with %d-token blocks" % bt)
        table, glens = pkv.pkv_block_table(cache, list(range(B)))
        assert [list(r[:len(p)]) for r, p in zip(table, planes)] == planes
        assert list(glens) == lens
        r_out, r_lse = o_att.decode_paged(q, kp, vp, dp.spec(), 1, planes, lens, HQ, by_plane=True)
        out, lse = gu.decode(dp, 1, q_dev, torch.from_numpy(table).cuda(), glens, HQ, 0)
        gu.assert_close(out.cpu().numpy(), r_out, "decode out, %d-token blocks" % bt)
        gu.assert_close(lse.cpu().numpy(), r_lse, "decode lse, %d-token blocks" % bt)
        outs[bt] = (out.cpu().numpy(), lse.cpu().numpy())
        pkv.pkv_cache_destroy(cache)
    assert np.array_equal(outs[16][0], outs[32][0]) and np.array_equal(outs[16][1], outs[32][1])
