"""The pool layout is the caller's, given by element strides: K and V in
separate allocations, head planes and blocks padded apart, a layer range
addressed through the pool descriptor.  Inject, append and decode through
such a pool must match the oracle (which reads the same strides) byte for
byte and within tolerance; a caller-chosen softmax scale and a call without
the log-sum-exp output are covered too."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,d,layout", [("bf16", 128, "padded"), ("f16", 64, "padded"),
                                            ("bf16", 128, "plane"), ("f16", 64, "plane")])
def test_padded_split_pool_inject_append_decode(dtype, d, layout):
    """layout "padded": head planes and blocks padded apart; "plane": one
    head's planes of consecutive blocks adjacent ([head][block] per layer,
    block stride one plane), as bench.py's plane layout."""
    import torch
    import paged_kv_cache_inject_amd as pkv
    from oracle import attention as o_att, inject as o_inject
    from oracle.allocator import AllocatorModel
    from oracle.layout import PoolSpec
    from oracle.rope import rope_table
    from tests import gpu_util as gu
    from workloads.configs import host_normal

    rng = np.random.default_rng(d)
    L, H, NB, HQ, max_pos = 3, 2, 20, 8, 512
    plane = 16 * d
    if layout == "plane":
        bs, hs = plane, NB * plane
        ls = H * hs
    else:
        hs = plane + 64                  # 128 bytes of padding after every head plane
        bs = H * hs + 128
        ls = NB * bs + 256
    total = L * ls
    fill = 0x7FAB
    k_buf = torch.full((total,), 0, dtype=torch.int16, device="cuda").fill_(fill).view(
        gu.torch_dtype(dtype))
    v_buf = torch.full((total,), 0, dtype=torch.int16, device="cuda").fill_(fill).view(
        gu.torch_dtype(dtype))
    spec = PoolSpec(L, NB, H, d, dtype, ls, bs, hs)
    desc = pkv.pkv_pool(L, NB, H, d, pkv.DTYPE_CODES[dtype], 0, k_buf.data_ptr(),
                        v_buf.data_ptr(), ls, bs, hs)
    k_ref = np.full(total, fill, dtype=np.uint16)
    v_ref = np.full(total, fill, dtype=np.uint16)

    cache = pkv.pkv_cache_create(NB, 3, 8, free_list_seed=9)
    model = AllocatorModel(NB, 3, 8, seed=9)
    for s, n in enumerate((70, 33, 100)):
        pkv.pkv_alloc_blocks(cache, s, n)
        model.alloc_blocks(s, n)
    n_src = 200
    src_k = host_normal(rng, (L, n_src, H, d), dtype)
    src_v = host_normal(rng, (L, n_src, H, d), dtype)
    dk = gu.to_device_raw(src_k.reshape(-1), dtype)
    dv = gu.to_device_raw(src_v.reshape(-1), dtype)
    src = pkv.make_src(dk, dv, n_src * H * d, H * d, n_src)
    o_cos, o_sin = rope_table(d, 10000.0, max_pos)
    _, _, dcos, dsin = gu.rope_tables(d, max_pos)
    runs = [(0, 70, 0, 0), (1, 33, 0, 70), (2, 100, 0, 100)]
    ws = gu.workspace(pkv.pkv_inject_workspace_bytes(runs))
    pkv.pkv_inject(cache, desc, src, runs, 0, L, "halves", dcos, dsin, max_pos, ws)
    lens = o_inject.inject(k_ref, v_ref, spec, model.tables, [0, 0, 0], runs, src_k.reshape(-1),
                           src_v.reshape(-1), n_src * H * d, H * d, 0, L, "halves", o_cos, o_sin)
    for s_, n_ in enumerate(lens):
        model.set_len(s_, n_)
    # append 5 tokens to every sequence, on every layer
    first = pkv.pkv_extend(cache, [0, 1, 2], 5)
    assert list(first) == model.extend([0, 1, 2], 5)
    table, glens = pkv.pkv_block_table(cache, [0, 1, 2])
    tdev = torch.from_numpy(table).cuda()
    fdev = torch.from_numpy(first.astype(np.int32)).cuda()
    keep = []
    for layer in range(L):
        kn = host_normal(rng, (3, 5, H, d), dtype)
        vn = host_normal(rng, (3, 5, H, d), dtype)
        kd = gu.to_device_raw(kn.reshape(-1), dtype)
        vd = gu.to_device_raw(vn.reshape(-1), dtype)
        keep.append((kd, vd))
        pkv.pkv_append_kv(desc, layer, tdev, fdev, 5, kd, vd, "halves", dcos, dsin, max_pos)
        o_inject.append(k_ref, v_ref, spec, layer, model.tables, model.lens, [0, 1, 2], 5, kn, vn,
                        "halves", o_cos, o_sin)
    torch.cuda.synchronize()
    gu.assert_bytes_equal(gu.raw_view(k_buf.cpu()), k_ref, "K buffer")
    gu.assert_bytes_equal(gu.raw_view(v_buf.cpu()), v_ref, "V buffer")

    q = host_normal(rng, (3, HQ, d), dtype)
    q_dev = gu.to_device_raw(q.reshape(-1), dtype).view(3, HQ, d)
    plan = pkv.pkv_decode_plan_create(glens, HQ, H, d, 0)
    dws = gu.workspace(pkv.pkv_decode_workspace_bytes(plan))
    pkv.pkv_decode_plan_upload(plan, dws)
    for layer in range(L):
        for scale in (0.0, 0.05):
            out = torch.full((3, HQ, d), float("nan"), device="cuda")
            lse = torch.full((3, HQ), float("nan"), device="cuda")
            use_lse = scale == 0.0
            pkv.pkv_decode_attention(plan, desc, layer, q_dev, tdev, out, lse if use_lse else None,
                                     dws, scale=scale)
            torch.cuda.synchronize()
            ref, ref_lse = o_att.decode_paged(q, k_ref, v_ref, spec, layer, model.tables,
                                              model.lens, HQ, by_plane=True,
                                              scale=None if scale == 0.0 else scale)
            gu.assert_close(out.cpu().numpy(), ref, "out layer %d scale %g" % (layer, scale))
            if use_lse:
                gu.assert_close(lse.cpu().numpy(), ref_lse, "lse layer %d" % layer)
            else:
                assert torch.isnan(lse).all()      # not written
    pkv.pkv_decode_plan_destroy(plan)
    # the same pool seen from its second layer on: layer 0 of this descriptor is layer 1
    eb = 2
    sub = pkv.pkv_pool(L - 1, NB, H, d, pkv.DTYPE_CODES[dtype], 0, k_buf.data_ptr() + ls * eb,
                       v_buf.data_ptr() + ls * eb, ls, bs, hs)
    out0, _ = _decode_desc(sub, 0, q_dev, tdev, glens, HQ, H, d)
    out1, _ = _decode_desc(desc, 1, q_dev, tdev, glens, HQ, H, d)
    assert torch.equal(out0, out1)
    pkv.pkv_cache_destroy(cache)


def _decode_desc(desc, layer, q_dev, tdev, lens, hq, h, d):
    import torch
    import paged_kv_cache_inject_amd as pkv
    from tests import gpu_util as gu
    plan = pkv.pkv_decode_plan_create(lens, hq, h, d, 0)
    ws = gu.workspace(pkv.pkv_decode_workspace_bytes(plan))
    pkv.pkv_decode_plan_upload(plan, ws)
    out = torch.empty(len(lens), hq, d, device="cuda")
    lse = torch.empty(len(lens), hq, device="cuda")
    pkv.pkv_decode_attention(plan, desc, layer, q_dev, tdev, out, lse, ws)
    torch.cuda.synchronize()
    pkv.pkv_decode_plan_destroy(plan)
    return out, lse
