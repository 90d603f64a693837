"""Shared blocks on the GPU against the oracle: random sequences of fork,
extend (copy-on-write, then the queued copies, then an append), inject into
shared blocks (copy-on-write inside the call), free, prefix match and commit,
with the whole pool compared byte for byte at checkpoints and decode over
the final tables within tolerance.  Also: chained copy queues carried out in
dependency levels equal the sequential reading, and beams forked from one
prompt decode like the prompt until they diverge."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


class Pair:
    """The library (device pool, allocator) and the oracle (host pool,
    allocator model) driven through the same operations."""

    def __init__(self, dtype, L=2, H=2, d=64, NB=32, S=5, MB=8, max_pos=256, seed=0, bt=16):
        import paged_kv_cache_inject_amd as pkv
        from oracle.allocator import AllocatorModel
        from oracle.rope import rope_table
        from tests import gpu_util as gu
        from workloads.configs import host_normal
        self.pkv, self.gu = pkv, gu
        self.rng = np.random.default_rng(seed)
        self.L, self.H, self.d, self.NB, self.S, self.MB = L, H, d, NB, S, MB
        self.bt, self.sub = bt, bt // 16                  # tokens per block, planes per block
        self.max_pos = max_pos
        self.dtype = dtype
        self.sdt = "bf16"
        fill = 0x5A if dtype == "fp8" else 0x7FAB
        self.dp = gu.DevicePool(L, NB * self.sub, H, d, dtype, fill_bits=fill)
        self.ks = self.vs = None
        if dtype == "fp8":
            self.ks = self.rng.uniform(0.004, 0.03, size=(L, H)).astype(np.float32)
            self.vs = self.rng.uniform(0.004, 0.03, size=(L, H)).astype(np.float32)
            self.dp.set_scales(self.ks, self.vs)
        self.ref = np.full(self.dp.total, fill, dtype=np.uint8 if dtype == "fp8" else np.uint16)
        self.kp, self.vp = self.dp.oracle_arrays(self.ref)
        self.cache = pkv.pkv_cache_create(NB, S, MB, free_list_seed=seed + 1, block_tokens=bt)
        self.m = AllocatorModel(NB, S, MB, seed=seed + 1, block_tokens=bt)
        self.o_cos, self.o_sin = rope_table(d, 10000.0, max_pos)
        _, _, self.dcos, self.dsin = gu.rope_tables(d, max_pos)
        self.n_src = 200
        self.src_k = host_normal(self.rng, (L, self.n_src, H, d), self.sdt)
        self.src_v = host_normal(self.rng, (L, self.n_src, H, d), self.sdt)
        self.dk = gu.to_device_raw(self.src_k.reshape(-1), self.sdt)
        self.dv = gu.to_device_raw(self.src_v.reshape(-1), self.sdt)
        self.src = pkv.make_src(self.dk, self.dv, self.n_src * H * d, H * d, self.n_src,
                                dtype=self.sdt)
        self.keep = []
        self.copies = 0                          # block copies carried out so far

    def planes(self):
        """The model's tables as rows of 16-token planes."""
        from oracle.allocator import expand_table
        return [expand_table(t, self.bt) for t in self.m.tables]

    # -- checks ----------------------------------------------------------------
    def check_host(self, what):
        pkv = self.pkv
        t, lens = pkv.pkv_block_table(self.cache, list(range(self.S)))
        got = [[int(x) for x in r] for r in t]
        want = [p + [-1] * (t.shape[1] - len(p)) for p in self.planes()]
        assert got == want, what
        assert list(lens) == self.m.lens, what
        assert pkv.pkv_free_list(self.cache) == list(self.m.free), what
        assert [pkv.pkv_block_refcount(self.cache, b) for b in range(self.NB)] == self.m.ref
        assert pkv.pkv_pending_copies(self.cache) == self.m.pending, what
        self.m.check_invariants()

    def check_pool(self, what):
        import torch
        torch.cuda.synchronize()
        self.gu.assert_bytes_equal(self.dp.host_copy(), self.ref, what)

    # -- operations --------------------------------------------------------------
    def flush(self):
        from oracle import inject as o_inject
        from oracle.allocator import expand_pairs
        self.pkv.pkv_copy_blocks(self.cache, self.dp.desc())
        pairs = self.m.take_pending()
        self.copies += len(pairs)
        o_inject.copy_blocks(self.kp, self.vp, self.dp.spec(), expand_pairs(pairs, self.bt))

    def extend_append(self, seqs, n):
        import torch
        from oracle import inject as o_inject
        from workloads.configs import host_normal
        pkv, gu = self.pkv, self.gu
        first = list(pkv.pkv_extend(self.cache, seqs, n))
        assert first == self.m.extend(seqs, n)
        self.check_host("after extend")
        self.flush()
        table, _ = pkv.pkv_block_table(self.cache, seqs)
        tdev = torch.from_numpy(table).cuda()
        fdev = torch.from_numpy(np.asarray(first, np.int32)).cuda()
        for layer in range(self.L):
            k_new = host_normal(self.rng, (len(seqs), n, self.H, self.d), self.sdt)
            v_new = host_normal(self.rng, (len(seqs), n, self.H, self.d), self.sdt)
            kd = gu.to_device_raw(k_new.reshape(-1), self.sdt)
            vd = gu.to_device_raw(v_new.reshape(-1), self.sdt)
            self.keep.append((kd, vd, tdev, fdev))
            pkv.pkv_append_kv(self.dp.desc(), layer, tdev, fdev, n, kd, vd, "pairs", self.dcos,
                              self.dsin, self.max_pos, new_dtype=self.sdt)
            o_inject.append(self.kp, self.vp, self.dp.spec(), layer, self.planes(), self.m.lens,
                            seqs, n, k_new, v_new, "pairs", self.o_cos, self.o_sin,
                            src_dtype=self.sdt, k_scale=self.ks, v_scale=self.vs)

    def inject(self, runs):
        from oracle import inject as o_inject
        pkv, gu = self.pkv, self.gu
        ws = gu.workspace(pkv.pkv_inject_workspace_bytes(runs))
        self.keep.append(ws)
        pkv.pkv_inject(self.cache, self.dp.desc(), self.src, runs, 0, self.L, "pairs", self.dcos,
                       self.dsin, self.max_pos, ws)
        from oracle.allocator import expand_pairs
        self.m.prepare_inject(runs)
        pairs = self.m.take_pending()
        self.copies += len(pairs)
        o_inject.copy_blocks(self.kp, self.vp, self.dp.spec(), expand_pairs(pairs, self.bt))
        lens = o_inject.inject(self.kp, self.vp, self.dp.spec(), self.planes(), self.m.lens, runs,
                               self.src_k.reshape(-1), self.src_v.reshape(-1),
                               self.n_src * self.H * self.d, self.H * self.d, 0, self.L, "pairs",
                               self.o_cos, self.o_sin, src_dtype=self.sdt, k_scale=self.ks,
                               v_scale=self.vs)
        for s, n in enumerate(lens):
            self.m.lens[s] = n

    def decode_all(self, hq):
        import torch
        from oracle import attention as o_att
        from workloads.configs import host_normal
        pkv, gu = self.pkv, self.gu
        seqs = list(range(self.S))
        table, lens = pkv.pkv_block_table(self.cache, seqs)
        q = host_normal(self.rng, (self.S, hq, self.d), "bf16")
        q_dev = gu.to_device_raw(q.reshape(-1), "bf16").view(q.shape)
        tdev = torch.from_numpy(table).cuda()
        for layer in range(self.L):
            ref, ref_lse = o_att.decode_paged(q, self.kp, self.vp, self.dp.spec(), layer,
                                              self.planes(), self.m.lens, hq, by_plane=True,
                                              q_dtype="bf16", k_scale=self.ks, v_scale=self.vs)
            out, lse = gu.decode(self.dp, layer, q_dev, tdev, lens, hq, 0, q_dtype="bf16")
            gu.assert_close(out.cpu().numpy(), ref, "decode out layer %d" % layer)
            gu.assert_close(lse.cpu().numpy(), ref_lse, "decode lse layer %d" % layer)


STEPS = 120


@pytest.mark.parametrize("dtype,seed,bt", [("bf16", 1, 16), ("bf16", 2, 16), ("fp8", 3, 16),
                                           ("bf16", 7, 32), ("fp8", 13, 32)])
def test_random_sharing_operations_pool_matches_oracle(dtype, seed, bt):
    from oracle.allocator import AllocError
    P = Pair(dtype, seed=seed, bt=bt)
    pkv, gu, m = P.pkv, P.gu, P.m
    rng = np.random.default_rng(1000 + seed)     # operation choices (data comes from P.rng)
    gu.say("sharing random ops", dtype, seed, "block", bt)
    history = []
    forks = hits = injects = 0
    for step in range(STEPS):
        op = rng.choice(["extend", "extend", "fork", "fork", "free", "inject", "match",
                         "commit"])
        s = int(rng.integers(0, P.S))
        try:
            if op == "extend":
                seqs = sorted(set(rng.integers(0, P.S, size=int(rng.integers(1, 3))).tolist()))
                n = int(rng.choice([1, 5, 16]))
                if any(m.lens[x] + n > P.MB * P.bt for x in seqs):
                    continue
                if sum(-(-(m.lens[x] + n) // P.bt) - len(m.tables[x]) + 1 for x in seqs) > len(m.free):
                    continue
                P.extend_append(seqs, n)
            elif op == "fork":
                empty = [x for x in range(P.S) if not m.tables[x] and x != s]
                if not empty or not m.tables[s]:
                    continue
                d = int(rng.choice(empty))
                pkv.pkv_fork(P.cache, s, d)
                m.fork(s, d)
                forks += 1
            elif op == "free":
                pkv.pkv_free_seq(P.cache, s)
                m.free_seq(s)
            elif op == "inject":
                if m.lens[s] == 0:
                    continue
                p0 = int(rng.integers(0, m.lens[s]))
                n = int(rng.integers(1, m.lens[s] - p0 + 1))
                src = int(rng.integers(0, P.n_src - n + 1))
                shared = sum(1 for i in range(p0 // P.bt, (p0 + n - 1) // P.bt + 1)
                             if m.ref[m.tables[s][i]] > 1)
                if shared > len(m.free):
                    continue
                P.inject([(s, n, p0, src)])
                injects += 1
            elif op == "match":
                if m.tables[s] or not history:
                    continue
                keys = list(history[int(rng.integers(0, len(history)))])
                want = m.prefix_match(s, keys)
                assert pkv.pkv_prefix_match(P.cache, s, keys) == want
                hits += want > 0
            else:
                if m.lens[s] < P.bt:
                    continue
                n_keys = int(rng.integers(P.bt, m.lens[s] + 1))
                keys = [int(x) for x in rng.integers(0, 1 << 62, size=n_keys)]
                em = ec = None
                try:
                    m.prefix_commit(s, keys)
                except AllocError as e:
                    em = e.code
                try:
                    pkv.pkv_prefix_commit(P.cache, s, keys)
                except pkv.PkvError as e:
                    ec = e.code
                assert ec == em, (ec, em)
                if em is None:
                    history.append(keys)
        finally:
            pass
        P.check_host("step %d %s" % (step, op))
        if step % 10 == 9:
            P.check_pool("pool after step %d" % step)
    P.flush()
    P.check_pool("final pool")
    gu.say("  forks %d injects %d prefix hits %d block copies %d"
           % (forks, injects, hits, P.copies))
    assert forks >= 4 and injects >= 6 and P.copies >= 5 and hits >= 1
    P.decode_all(hq=4)
    pkv.pkv_cache_destroy(P.cache)


def test_chained_copy_queue_equals_sequential_copies():
    """A queue whose copies depend on one another (a block copied again after
    it received a copy; a block that was read being overwritten) must end as
    if carried out one after another."""
    P = Pair("bf16", NB=12, S=4, MB=4, seed=9)
    pkv, m = P.pkv, P.m
    P.extend_append([0], 20)                 # blocks a, b (b half full)
    pkv.pkv_fork(P.cache, 0, 1)
    m.fork(0, 1)
    assert list(pkv.pkv_extend(P.cache, [1], 1)) == m.extend([1], 1)   # b -> x queued
    pkv.pkv_fork(P.cache, 1, 2)
    m.fork(1, 2)
    assert list(pkv.pkv_extend(P.cache, [2], 1)) == m.extend([2], 1)   # x -> y: reads a copy's target
    pend = pkv.pkv_pending_copies(P.cache)
    assert pend == m.pending and len(pend) == 2 and pend[1][0] == pend[0][1]
    P.check_host("chained queue")
    P.flush()
    P.check_pool("pool after chained copies")
    pkv.pkv_cache_destroy(P.cache)


def test_forked_beams_decode_like_the_prompt_until_they_diverge():
    import torch
    P = Pair("bf16", L=1, H=2, d=128, NB=40, S=4, MB=8, seed=5)
    pkv, gu, m = P.pkv, P.gu, P.m
    P.extend_append([0], 70)
    for b in (1, 2, 3):
        pkv.pkv_fork(P.cache, 0, b)
        m.fork(0, b)
    table, lens = pkv.pkv_block_table(P.cache, [0, 1, 2, 3], P.MB)
    q1 = gu.to_device_raw(np.tile(np.random.default_rng(1).standard_normal((1, 8, 128))
                                  .astype(np.float32).view(np.uint32) >> 16, (4, 1, 1))
                          .astype(np.uint16).reshape(-1), "bf16").view(4, 8, 128)
    out, lse = gu.decode(P.dp, 0, q1, torch.from_numpy(table).cuda(), lens, 8, 0, q_dtype="bf16")
    o = out.cpu().numpy()
    for b in (1, 2, 3):                       # same blocks, same query: bit-identical
        assert np.array_equal(o[b], o[0])
    P.extend_append([1, 2, 3], 1)             # three beams copy the shared last block
    assert sum(1 for x in set(b for t in m.tables for b in t) if m.ref[x] == 4) == 4
    P.extend_append([0], 1)
    P.check_pool("pool after beams diverge")
    P.decode_all(hq=8)
    pkv.pkv_cache_destroy(P.cache)
