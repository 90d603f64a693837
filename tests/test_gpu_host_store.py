"""A source store in pinned host memory ([InferScale] §6: the pre-RoPE store
kept in pinned host DRAM, the retrieved rows streamed over PCIe): the inject
kernel reads it directly over PCIe.  The pool must come out byte for byte as
the oracle's (bf16 and fp8 pools), and as the same inject from a device
store at the reduced injection-workload size."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


class HostStore:
    """K and V stores of [layers][tokens][heads][d] raw elements in pinned
    host memory from pkv_host_alloc."""

    def __init__(self, k_raw, v_raw):
        import paged_kv_cache_inject_amd as pkv
        self.pkv = pkv
        self.nbytes = k_raw.nbytes
        self.k = pkv.pkv_host_alloc(self.nbytes)
        self.v = pkv.pkv_host_alloc(self.nbytes)
        pkv.host_view(self.k, self.nbytes)[:] = np.ascontiguousarray(k_raw).view(np.uint8).reshape(-1)
        pkv.host_view(self.v, self.nbytes)[:] = np.ascontiguousarray(v_raw).view(np.uint8).reshape(-1)

    def free(self):
        self.pkv.pkv_host_free(self.k)
        self.pkv.pkv_host_free(self.v)


@pytest.mark.parametrize("pool_dtype,d,mode", [("bf16", 128, "pairs"), ("bf16", 64, "halves"),
                                               ("fp8", 128, "pairs")])
def test_inject_from_pinned_host_store_matches_oracle(pool_dtype, d, mode):
    import torch
    import paged_kv_cache_inject_amd as pkv
    from oracle import inject as o_inject
    from oracle.allocator import AllocatorModel
    from oracle.rope import rope_table
    from tests import gpu_util as gu
    from workloads.configs import host_normal

    gu.say("host-store inject", pool_dtype, d, mode)
    rng = np.random.default_rng(d + len(mode))
    L, H, NB, max_pos = 3, 4, 48, 400
    fill = 0x5A if pool_dtype == "fp8" else 0x7FAB
    dp = gu.DevicePool(L, NB, H, d, pool_dtype, fill_bits=fill)
    ks = vs = None
    if pool_dtype == "fp8":
        ks = rng.uniform(0.004, 0.03, size=(L, H)).astype(np.float32)
        vs = rng.uniform(0.004, 0.03, size=(L, H)).astype(np.float32)
        dp.set_scales(ks, vs)
    cache = pkv.pkv_cache_create(NB, 4, 16, free_list_seed=3)
    model = AllocatorModel(NB, 4, 16, seed=3)
    for s, n in enumerate((120, 37, 250, 16)):
        pkv.pkv_alloc_blocks(cache, s, n)
        model.alloc_blocks(s, n)
    n_src = 300
    src_k = host_normal(rng, (L, n_src, H, d), "bf16")
    src_v = host_normal(rng, (L, n_src, H, d), "bf16")
    store = HostStore(src_k, src_v)
    try:
        src = pkv.make_src(store.k, store.v, n_src * H * d, H * d, n_src, dtype="bf16")
        o_cos, o_sin = rope_table(d, 10000.0, max_pos)
        _, _, dcos, dsin = gu.rope_tables(d, max_pos)
        ref = np.full(dp.total, fill, dtype=np.uint8 if pool_dtype == "fp8" else np.uint16)
        kp, vp = dp.oracle_arrays(ref)
        lens = [0] * 4
        for i, runs in enumerate([[(0, 120, 0, 0), (1, 37, 0, 120), (3, 16, 0, 157)],
                                  [(2, 5, 3, 200), (2, 40, 9, 173), (2, 100, 60, 13),
                                   (0, 24, 40, 276)]]):
            ws = gu.workspace(pkv.pkv_inject_workspace_bytes(runs))
            pkv.pkv_inject(cache, dp.desc(), src, runs, 0, L, mode, dcos, dsin, max_pos, ws)
            torch.cuda.synchronize()
            lens = o_inject.inject(kp, vp, dp.spec(), model.tables, lens, runs, src_k.reshape(-1),
                                   src_v.reshape(-1), n_src * H * d, H * d, 0, L, mode, o_cos,
                                   o_sin, src_dtype="bf16", k_scale=ks, v_scale=vs)
            gu.assert_bytes_equal(dp.host_copy(), ref, "pool after host-store inject %d" % i)
    finally:
        torch.cuda.synchronize()
        store.free()
        pkv.pkv_cache_destroy(cache)


def test_reduced_workload_host_store_equals_device_store():
    import torch
    import paged_kv_cache_inject_amd as pkv
    from tests import gpu_util as gu
    from workloads.configs import INJECT_TOP8, inject_structure, device_normal

    cfg = INJECT_TOP8
    st = inject_structure(cfg, n_chunks=120, batch=8)
    L, H, d = cfg.n_layers, cfg.n_kv_heads, cfg.head_dim
    n_src, row = st["n_src"], H * d
    gu.say("host-store workload: %d source tokens, %d runs" % (n_src, len(st["runs"])))
    dev_k = torch.empty(L * n_src * row, dtype=torch.bfloat16, device="cuda")
    dev_v = torch.empty(L * n_src * row, dtype=torch.bfloat16, device="cuda")
    for layer in range(L):
        a, b = layer * n_src * row, (layer + 1) * n_src * row
        dev_k[a:b] = device_normal(b - a, "bf16", cfg.seed * 1000 + 2 * layer)
        dev_v[a:b] = device_normal(b - a, "bf16", cfg.seed * 1000 + 2 * layer + 1)
    nbytes = dev_k.numel() * 2
    hk, hv = pkv.pkv_host_alloc(nbytes), pkv.pkv_host_alloc(nbytes)
    try:
        # device -> torch-owned host tensor, then a plain host copy into the
        # library's pinned buffers (torch never copies into memory it did not
        # allocate)
        for addr, t in ((hk, dev_k), (hv, dev_v)):
            host = t.view(torch.uint8).cpu().numpy()
            assert host.nbytes == nbytes
            pkv.host_view(addr, nbytes)[:] = host
            del host
        max_pos = 4096
        _, _, dcos, dsin = gu.rope_tables(d, max_pos)
        pools = []
        for k, v in ((dev_k, dev_v), (hk, hv)):
            dp = gu.DevicePool(L, st["num_blocks"], H, d, "bf16", fill_bits=0x7FAB)
            cache = pkv.pkv_cache_create(st["num_blocks"], 8, st["max_blocks"], st["free_list_seed"])
            for b_, m in enumerate(st["mem_lens"]):
                pkv.pkv_alloc_blocks(cache, b_, int(m))
            src = pkv.make_src(k, v, n_src * row, row, n_src, dtype="bf16")
            ws = gu.workspace(pkv.pkv_inject_workspace_bytes(st["runs"]))
            pkv.pkv_inject(cache, dp.desc(), src, st["runs"], 0, L, "pairs", dcos, dsin, max_pos, ws)
            torch.cuda.synchronize()
            pools.append(dp)
            pkv.pkv_cache_destroy(cache)
        assert torch.equal(pools[0].buf.view(torch.int16), pools[1].buf.view(torch.int16))
    finally:
        torch.cuda.synchronize()
        pkv.pkv_host_free(hk)
        pkv.pkv_host_free(hv)
