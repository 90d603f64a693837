"""One decode step in one launch (pkv_append_decode_attention): every
sequence's newest token is written at position len - 1 (K rotated at that
position, V as given) and attended to ([KV essay] "The fix"; [InferScale] §2).
The call must leave the pool and produce out/lse byte for byte as
pkv_append_kv (first position len - 1, one token) followed by
pkv_decode_attention does, and match the oracle's append and decode: pool
bytes exactly, attention within tolerance.  Cases cover the MFMA kernel
(bf16, f16, fp8 pools; head dims 64 and 128; 1, 2 and 4 tiles of 16 query
heads per KV head), the generic kernel (float32 pools), split ranges (only
the last range writes), a sliding window, the three rotary pairings, and
lengths 0, 1 and block edges."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

LENS = [0, 1, 15, 16, 17, 33, 100, 257, 700, 2000]

CASES = [
    # pool dtype, query heads, KV heads, head dim, rotary pairing, part tokens, window
    ("bf16", 64, 8, 128, "pairs", 0, 0),
    ("bf16", 32, 4, 128, "halves", 16, 0),
    ("f16", 8, 8, 64, "halves", 0, 0),
    ("f16", 16, 2, 64, "none", 32, 0),
    ("fp8", 16, 2, 128, "halves", 0, 0),
    ("fp8", 8, 2, 64, "halves", 16, 0),
    ("fp8", 4, 4, 64, "pairs", 0, 0),
    ("f32", 4, 2, 64, "pairs", 0, 0),
    ("bf16", 64, 2, 128, "halves", 0, 0),
    ("fp8", 64, 2, 128, "pairs", 16, 0),
    ("bf16", 64, 1, 64, "halves", 0, 0),
    ("bf16", 32, 8, 128, "pairs", 0, 100),
    # fp8 with scales per (layer, block, KV head)
    ("fp8b", 16, 2, 128, "pairs", 0, 0), ("fp8b", 64, 1, 64, "halves", 16, 0),
]


def _fill(dp, rng, dtype):
    """Random pool contents (finite codes for fp8); returns the raw host copy."""
    from tests import gpu_util as gu
    from workloads.configs import host_normal
    if dtype == "fp8":
        codes = rng.integers(0, 0x70, size=dp.total, dtype=np.uint8)
        raw = codes | (rng.integers(0, 2, size=dp.total, dtype=np.uint8) << 7).astype(np.uint8)
    else:
        raw = host_normal(rng, (dp.total,), dtype)
    dp.buf.copy_(gu.to_device_raw(raw, dtype))
    return raw.copy()


@pytest.mark.parametrize("dtype,hq,hkv,d,mode,part,window", CASES)
def test_append_decode_matches_two_calls_and_oracle(dtype, hq, hkv, d, mode, part, window):
    import torch
    import paged_kv_cache_inject_amd as pkv
    from oracle import attention as o_att, inject as o_inject
    from oracle.rope import rope_table
    from tests import gpu_util as gu
    from workloads.configs import host_normal, deal_tables

    gu.say("append+decode", dtype, hq, hkv, d, mode, part, window)
    rng = np.random.default_rng(hq * 1009 + hkv * 31 + d + part + window + (dtype == "fp8b"))
    blockwise = dtype == "fp8b"
    dtype = "fp8" if blockwise else dtype
    L, layer = 2, 1
    lens = np.array(LENS, dtype=np.int64)
    B = len(lens)
    need = int(sum(-(-int(x) // 16) for x in lens))
    nb = need + 5
    table = deal_tables(rng.permutation(nb)[:need].astype(np.int32), lens, 128)
    tdev = torch.from_numpy(table).cuda()
    pools = [gu.DevicePool(L, nb, hkv, d, dtype) for _ in range(2)]
    ks = vs = None
    if dtype == "fp8":
        shape = (L, nb, hkv) if blockwise else (L, hkv)
        ks = rng.uniform(0.01, 0.03, size=shape).astype(np.float32)
        vs = rng.uniform(0.01, 0.03, size=shape).astype(np.float32)
        for dp in pools:
            dp.set_scales(ks, vs)
    raw = _fill(pools[0], rng, dtype)
    pools[1].buf.copy_(pools[0].buf)
    qdt = "bf16" if dtype == "fp8" else dtype
    q = host_normal(rng, (B, hq, d), qdt)
    k_new = host_normal(rng, (B, hkv, d), qdt)
    v_new = host_normal(rng, (B, hkv, d), qdt)
    q_dev = gu.to_device_raw(q.reshape(-1), qdt).view(B, hq, d)
    kd = gu.to_device_raw(k_new.reshape(-1), qdt)
    vd = gu.to_device_raw(v_new.reshape(-1), qdt)
    max_pos = int(lens.max())
    o_cos, o_sin = rope_table(d, 10000.0, max_pos)
    _, _, dcos, dsin = gu.rope_tables(d, max_pos)

    # two calls: append at len - 1 (a length-0 sequence gets -1: no write), then decode
    first = torch.from_numpy((lens - 1).astype(np.int32)).cuda()
    pkv.pkv_append_kv(pools[0].desc(), layer, tdev, first, 1, kd, vd, mode, dcos, dsin, max_pos,
                      new_dtype=qdt)
    out_a, lse_a = gu.decode(pools[0], layer, q_dev, tdev, lens, hq, part, q_dtype=qdt,
                             window=window)

    # one call
    plan = pkv.pkv_decode_plan_create(lens, hq, hkv, d, part, window=window)
    ws = gu.workspace(pkv.pkv_decode_workspace_bytes(plan))
    pkv.pkv_decode_plan_upload(plan, ws)
    out_b = torch.full((B, hq, d), float("nan"), device="cuda")
    lse_b = torch.full((B, hq), float("nan"), device="cuda")
    pkv.pkv_append_decode_attention(plan, pools[1].desc(), layer, q_dev, tdev, kd, vd, mode, dcos,
                                    dsin, max_pos, out_b, lse_b, ws, q_dtype=qdt)
    torch.cuda.synchronize()
    pkv.pkv_decode_plan_destroy(plan)

    got_pool = pools[1].host_copy()
    gu.assert_bytes_equal(got_pool, pools[0].host_copy(), "pool: one call vs two calls")
    assert torch.equal(out_b, out_a), "out: one call vs two calls"
    assert torch.equal(lse_b, lse_a), "lse: one call vs two calls"

    kp, vp = pools[1].oracle_arrays(raw)
    seqs = [b for b in range(B) if lens[b] > 0]
    o_inject.append(kp, vp, pools[1].spec(), layer, [list(r) for r in table], lens, seqs, 1,
                    k_new[seqs][:, None], v_new[seqs][:, None], mode, o_cos, o_sin,
                    src_dtype=qdt, k_scale=ks, v_scale=vs)
    gu.assert_bytes_equal(got_pool, raw, "pool vs oracle append")
    ref, ref_lse = o_att.decode_paged(q, kp, vp, pools[1].spec(), layer,
                                      [list(r) for r in table], lens, hq, by_plane=True,
                                      q_dtype=qdt, k_scale=ks, v_scale=vs, window=window or None)
    gu.assert_close(out_b.cpu().numpy(), ref, "out vs oracle")
    gu.assert_close(lse_b.cpu().numpy(), ref_lse, "lse vs oracle")


def test_append_decode_length_one_returns_the_new_value():
    """A sequence holding only the new token attends to it alone: out is its
    V row (as stored: exact for 16-bit pools) and lse is its scaled score
    against the key stored rotated by R_0 = I."""
    import torch
    import paged_kv_cache_inject_amd as pkv
    from tests import gpu_util as gu
    from workloads.configs import host_normal
    from oracle.numerics import to_f64

    rng = np.random.default_rng(77)
    hq, hkv, d = 16, 4, 128
    lens = np.array([1, 1, 1], dtype=np.int64)
    dp = gu.DevicePool(1, 8, hkv, d, "bf16", fill_bits=0x7FC1)     # NaN everywhere else
    table = np.array([[5], [0], [7]], dtype=np.int32)
    tdev = torch.from_numpy(table).cuda()
    q = host_normal(rng, (3, hq, d), "bf16")
    k_new = host_normal(rng, (3, hkv, d), "bf16")
    v_new = host_normal(rng, (3, hkv, d), "bf16")
    q_dev = gu.to_device_raw(q.reshape(-1), "bf16").view(3, hq, d)
    kd = gu.to_device_raw(k_new.reshape(-1), "bf16")
    vd = gu.to_device_raw(v_new.reshape(-1), "bf16")
    _, _, dcos, dsin = gu.rope_tables(d, 4)
    plan = pkv.pkv_decode_plan_create(lens, hq, hkv, d, 0)
    ws = gu.workspace(pkv.pkv_decode_workspace_bytes(plan))
    pkv.pkv_decode_plan_upload(plan, ws)
    out = torch.empty(3, hq, d, device="cuda")
    lse = torch.empty(3, hq, device="cuda")
    pkv.pkv_append_decode_attention(plan, dp.desc(), 0, q_dev, tdev, kd, vd, "pairs", dcos, dsin,
                                    4, out, lse, ws)
    torch.cuda.synchronize()
    pkv.pkv_decode_plan_destroy(plan)
    o, ls = out.cpu().numpy(), lse.cpu().numpy()
    g = hq // hkv
    # every other slot of the written blocks (and every other block) keeps its bits
    pool = dp.host_copy()
    written = np.zeros(dp.total, dtype=bool)
    for b in range(3):
        for h in range(hkv):
            base = int(table[b, 0]) * dp.block_stride + h * dp.head_stride
            for c in range(d // 8):                     # K: chunk-major, slot 0
                written[base + c * 16 * 8: base + c * 16 * 8 + 8] = True
            written[dp.v_off + base + np.arange(d) * 16] = True   # V: dim-major, slot 0
    assert (pool[~written] == 0x7FC1).all()
    assert not (pool[written] == 0x7FC1).any()
    for b in range(3):
        for h in range(hq):
            v = to_f64(v_new[b, h // g], "bf16")
            k = to_f64(k_new[b, h // g], "bf16")
            assert np.array_equal(o[b, h], v.astype(np.float32))
            s = float(k @ to_f64(q[b, h], "bf16")) / np.sqrt(d)
            assert abs(ls[b, h] - s) <= 1e-3 + 2e-3 * abs(s)


NAN_BITS = {"bf16": 0x7FC1, "f16": 0x7E01, "fp8": 0x7F, "f32": 0x7FC00000}


@pytest.mark.parametrize("dtype,hq,hkv,d,part", [
    ("bf16", 64, 8, 128, 0), ("bf16", 64, 8, 128, 16), ("fp8", 16, 2, 128, 0),
    ("bf16", 32, 1, 128, 48), ("f16", 8, 8, 64, 16), ("f32", 4, 2, 64, 0),
])
def test_out_of_range_block_ids_are_skipped(dtype, hq, hkv, d, part):
    """Table entries that name no block (negative, or >= num_blocks) inside a
    sequence's length: the newest token is not written when its block is one
    of them, those positions drop out of the attention, and a sequence left
    with none gives 0 / -inf.  The kernels read block 0 in their place and
    mask it; block 0 holds NaN here, so a leak would show.  Both the one-call
    step and the two calls, split or not, against the oracle."""
    import torch
    import paged_kv_cache_inject_amd as pkv
    from oracle import attention as o_att, inject as o_inject
    from oracle.rope import rope_table
    from tests import gpu_util as gu
    from workloads.configs import host_normal, deal_tables

    gu.say("out-of-range block ids", dtype, hq, hkv, d, part)
    rng = np.random.default_rng(hq * 7 + hkv + d + part)
    L, layer = 2, 1
    lens = np.array(LENS, dtype=np.int64)
    B = len(lens)
    need = int(sum(-(-int(x) // 16) for x in lens))
    nb = need + 5
    # block 0 is never dealt: the kernels' stand-in for a rejected id
    table = deal_tables((1 + rng.permutation(nb - 1)[:need]).astype(np.int32), lens, 128)
    table[1, 0] = nb                  # len 1: its only block (the new token's)
    table[4, 0] = -1                  # len 17: the block before the new token's
    table[6, 6] = -(2 ** 31)          # len 100: the newest token's block
    table[8, 20] = nb + 999           # len 700: a middle block
    table[9, 0], table[9, 60] = -2, 10 ** 9
    tdev = torch.from_numpy(table).cuda()
    pools = [gu.DevicePool(L, nb, hkv, d, dtype) for _ in range(2)]
    ks = vs = None
    if dtype == "fp8":
        ks = rng.uniform(0.01, 0.03, size=(L, hkv)).astype(np.float32)
        vs = rng.uniform(0.01, 0.03, size=(L, hkv)).astype(np.float32)
        for dp in pools:
            dp.set_scales(ks, vs)
    raw = _fill(pools[0], rng, dtype)
    for lay in range(L):
        a = lay * pools[0].layer_stride
        raw[a:a + pools[0].block_stride] = NAN_BITS[dtype]
    pools[0].buf.copy_(gu.to_device_raw(raw, dtype))
    pools[1].buf.copy_(pools[0].buf)
    qdt = "bf16" if dtype == "fp8" else dtype
    q = host_normal(rng, (B, hq, d), qdt)
    k_new = host_normal(rng, (B, hkv, d), qdt)
    v_new = host_normal(rng, (B, hkv, d), qdt)
    q_dev = gu.to_device_raw(q.reshape(-1), qdt).view(B, hq, d)
    kd = gu.to_device_raw(k_new.reshape(-1), qdt)
    vd = gu.to_device_raw(v_new.reshape(-1), qdt)
    max_pos = int(lens.max())
    o_cos, o_sin = rope_table(d, 10000.0, max_pos)
    _, _, dcos, dsin = gu.rope_tables(d, max_pos)

    first = torch.from_numpy((lens - 1).astype(np.int32)).cuda()
    pkv.pkv_append_kv(pools[0].desc(), layer, tdev, first, 1, kd, vd, "pairs", dcos, dsin,
                      max_pos, new_dtype=qdt)
    out_a, lse_a = gu.decode(pools[0], layer, q_dev, tdev, lens, hq, part, q_dtype=qdt)
    plan = pkv.pkv_decode_plan_create(lens, hq, hkv, d, part)
    ws = gu.workspace(pkv.pkv_decode_workspace_bytes(plan))
    pkv.pkv_decode_plan_upload(plan, ws)
    out_b = torch.full((B, hq, d), float("nan"), device="cuda")
    lse_b = torch.full((B, hq), float("nan"), device="cuda")
    pkv.pkv_append_decode_attention(plan, pools[1].desc(), layer, q_dev, tdev, kd, vd, "pairs",
                                    dcos, dsin, max_pos, out_b, lse_b, ws, q_dtype=qdt)
    torch.cuda.synchronize()
    pkv.pkv_decode_plan_destroy(plan)

    got_pool = pools[1].host_copy()
    gu.assert_bytes_equal(got_pool, pools[0].host_copy(), "pool: one call vs two calls")
    assert torch.equal(out_b, out_a), "out: one call vs two calls"
    assert torch.equal(lse_b, lse_a), "lse: one call vs two calls"

    kp, vp = pools[1].oracle_arrays(raw)
    rows = [list(r) for r in table]
    seqs = [b for b in range(B) if lens[b] > 0]
    o_inject.append(kp, vp, pools[1].spec(), layer, rows, lens, seqs, 1, k_new[seqs][:, None],
                    v_new[seqs][:, None], "pairs", o_cos, o_sin, src_dtype=qdt, k_scale=ks,
                    v_scale=vs, num_blocks=nb)
    gu.assert_bytes_equal(got_pool, raw, "pool vs oracle append")
    ref, ref_lse = o_att.decode_paged(q, kp, vp, pools[1].spec(), layer, rows, lens, hq,
                                      q_dtype=qdt, k_scale=ks, v_scale=vs, num_blocks=nb)
    o, ls = out_b.cpu().numpy(), lse_b.cpu().numpy()
    assert np.all(o[1] == 0) and np.all(np.isneginf(ls[1])), "a sequence with no block left"
    gu.assert_close(o, ref, "out vs oracle")
    gu.assert_close(ls, ref_lse, "lse vs oracle")
