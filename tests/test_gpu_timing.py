"""The kernel-timing measurement helper: with pkv_kernel_timing on, every
decode launch records its own duration; the durations come back in launch
order, each positive, together no longer than the wall time around them, and
timing changes no result."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def test_kernel_timing_records_each_decode_launch():
    import torch
    import paged_kv_cache_inject_amd as pkv
    from tests import gpu_util as gu
    from workloads.configs import host_normal, deal_tables

    rng = np.random.default_rng(5)
    lens = np.array([300, 1000, 17, 0, 4096], dtype=np.int64)
    hq, hkv, d = 16, 4, 128
    need = int(sum(-(-int(x) // 16) for x in lens))
    table = deal_tables(rng.permutation(need + 3)[:need].astype(np.int32), lens, 256)
    dp = gu.DevicePool(1, need + 3, hkv, d, "bf16")
    dp.buf.copy_(gu.to_device_raw(host_normal(rng, (dp.total,), "bf16"), "bf16"))
    q = host_normal(rng, (len(lens), hq, d), "bf16")
    q_dev = gu.to_device_raw(q.reshape(-1), "bf16").view(len(lens), hq, d)
    tdev = torch.from_numpy(table).cuda()
    plan = pkv.pkv_decode_plan_create(lens, hq, hkv, d, 0)
    ws = gu.workspace(pkv.pkv_decode_workspace_bytes(plan))
    pkv.pkv_decode_plan_upload(plan, ws)
    out0 = torch.empty(len(lens), hq, d, device="cuda")
    lse0 = torch.empty(len(lens), hq, device="cuda")
    pkv.pkv_decode_attention(plan, dp.desc(), 0, q_dev, tdev, out0, lse0, ws)
    torch.cuda.synchronize()
    assert len(pkv.pkv_kernel_times()) == 0          # nothing recorded while off

    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    outs = []
    pkv.pkv_kernel_timing(True)
    try:
        s.record()
        for _ in range(5):
            out = torch.empty_like(out0)
            lse = torch.empty_like(lse0)
            pkv.pkv_decode_attention(plan, dp.desc(), 0, q_dev, tdev, out, lse, ws)
            outs.append((out, lse))
        e.record()
        torch.cuda.synchronize()
    finally:
        pkv.pkv_kernel_timing(False)
    times = pkv.pkv_kernel_times()
    assert len(times) == 5
    assert (times > 0).all()
    assert times.sum() <= s.elapsed_time(e) * 1.01
    for out, lse in outs:
        assert torch.equal(out, out0) and torch.equal(lse, lse0)
    assert len(pkv.pkv_kernel_times()) == 0          # released
    pkv.pkv_decode_plan_destroy(plan)
