"""The allocation-free decode step (pkv_append_decode_attention_noalloc,
for callers that cannot allocate): on calls in a row, each with a smaller
input than the one before, its pool writes, out and lse equal those of
pkv_append_decode_attention with a caller workspace, byte for byte; a plan
whose workspace exceeds the static scratch is refused before anything is
enqueued."""

import numpy as np
import pytest
import torch  # noqa: F401  (torch's HIP runtime is loaded before the library binds to it)


def test_plan_beyond_the_static_scratch_is_refused():
    """Host-side check only (fake device pointers, never touched)."""
    import paged_kv_cache_inject_amd as pkv
    fake = 1 << 20
    pool = pkv.pkv_pool(1, 8, 8, 128, pkv.PKV_BF16, 0, fake, fake + 4096, 8 * 4096, 4096, 1024)
    plan = pkv.pkv_decode_plan_create([16384] * 8, 64, 8, 128, 16)
    try:
        assert pkv.pkv_decode_workspace_bytes(plan) > pkv.PKV_NOALLOC_SCRATCH_BYTES
        tables = np.zeros((8, 1024), dtype=np.int32)
        with pytest.raises(pkv.PkvError) as e:
            pkv.pkv_append_decode_attention_noalloc(plan, pool, 0, fake, tables, fake, fake,
                                                    "pairs", fake, fake, 16384, fake, fake,
                                                    stream=0, q_dtype="bf16")
        assert e.value.code == "WORKSPACE" and "static scratch" in str(e.value)
    finally:
        pkv.pkv_decode_plan_destroy(plan)


def _one_call_pair(dtype, hq, hkv, d, lens, part, mode, seed):
    """The same decode step through both entry points on two copies of one
    pool; returns nothing, asserts byte equality."""
    import torch
    import paged_kv_cache_inject_amd as pkv
    from tests import gpu_util as gu
    from workloads.configs import host_normal, deal_tables, device_normal

    gu.say("no-alloc step", dtype, hq, hkv, d, list(lens), part, mode)
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, dtype=np.int64)
    B = len(lens)
    need = int(sum(-(-int(x) // 16) for x in lens))
    nb = need + 3
    table = deal_tables(rng.permutation(nb)[:need].astype(np.int32), lens, 512)
    tdev = torch.from_numpy(table).cuda()
    pools = [gu.DevicePool(2, nb, hkv, d, dtype) for _ in range(2)]
    pools[0].buf.copy_(device_normal(pools[0].total, dtype, seed))
    pools[1].buf.copy_(pools[0].buf)
    q = host_normal(rng, (B, hq, d), dtype)
    k_new = host_normal(rng, (B, hkv, d), dtype)
    v_new = host_normal(rng, (B, hkv, d), dtype)
    q_dev = gu.to_device_raw(q.reshape(-1), dtype).view(B, hq, d)
    kd = gu.to_device_raw(k_new.reshape(-1), dtype)
    vd = gu.to_device_raw(v_new.reshape(-1), dtype)
    max_pos = int(lens.max()) + 1
    _, _, dcos, dsin = gu.rope_tables(d, max_pos)
    plan = pkv.pkv_decode_plan_create(lens, hq, hkv, d, part)
    try:
        assert pkv.pkv_decode_workspace_bytes(plan) <= pkv.PKV_NOALLOC_SCRATCH_BYTES
        ws = gu.workspace(pkv.pkv_decode_workspace_bytes(plan))
        pkv.pkv_decode_plan_upload(plan, ws)
        outs = []
        for i in range(2):
            out = torch.full((B, hq, d), float("nan"), device="cuda")
            lse = torch.full((B, hq), float("nan"), device="cuda")
            if i == 0:
                pkv.pkv_append_decode_attention(plan, pools[0].desc(), 1, q_dev, tdev, kd, vd, mode,
                                                dcos, dsin, max_pos, out, lse, ws)
            else:
                pkv.pkv_append_decode_attention_noalloc(plan, pools[1].desc(), 1, q_dev, tdev, kd,
                                                        vd, mode, dcos, dsin, max_pos, out, lse)
            outs.append((out, lse))
        torch.cuda.synchronize()
    finally:
        pkv.pkv_decode_plan_destroy(plan)
    assert torch.equal(outs[0][0], outs[1][0]), "out: no-alloc vs workspace"
    assert torch.equal(outs[0][1], outs[1][1]), "lse: no-alloc vs workspace"
    gu.assert_bytes_equal(pools[1].host_copy(), pools[0].host_copy(), "pool: no-alloc vs workspace")
    assert not torch.isnan(outs[1][0][lens > 0]).any()


@pytest.mark.gpu
def test_noalloc_step_equals_workspace_step_on_two_calls():
    # a launch of 16 workgroups per CU or more (128 sequences x 32 KV heads,
    # one empty): the step appends in a launch of its own, from the newest
    # positions the call copies into the scratch
    lens = np.random.default_rng(13).integers(520, 700, size=128)
    lens[5] = 0
    _one_call_pair("f16", 32, 32, 128, lens.tolist(), 0, "pairs", 13)
    # split sequences (partial states and the merge use the scratch)
    _one_call_pair("bf16", 32, 8, 128, [3000, 17, 1, 0, 900, 2048, 5000, 600], 512, "pairs", 11)
    # second call, smaller: fewer, shorter sequences, another format; the scratch
    # still holds the first call's work list and partials
    _one_call_pair("f16", 8, 4, 64, [40, 700, 16], 0, "halves", 12)
