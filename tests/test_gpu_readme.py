"""The README's quick start runs as printed, and what it computes is what the
oracle computes: the injected and appended pool byte for byte, and the last
layer's attention within tolerance."""

import os
import re

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _quickstart():
    text = open(os.path.join(ROOT, "README.md")).read()
    m = re.search(r"<!-- quickstart -->\s*```python\n(.*?)```\s*<!-- /quickstart -->", text, re.S)
    assert m, "quick start block not found"
    return m.group(1)


def test_readme_quickstart_runs_and_matches_the_oracle():
    import torch
    from oracle import attention as o_att, inject as o_inject
    from oracle.allocator import AllocatorModel
    from oracle.layout import PoolSpec
    from oracle.rope import rope_table
    from tests import gpu_util as gu

    code = _quickstart()
    # keep what the snippet draws, to replay it on the oracle
    drawn = []
    real_randn = torch.randn

    def randn(*a, **k):
        t = real_randn(*a, **k)
        drawn.append(t)
        return t

    torch.manual_seed(0)
    ns = {}
    torch.randn = randn
    try:
        exec(compile(code, "README quick start", "exec"), ns)
    finally:
        torch.randn = real_randn
    L, H, D, HQ, NB, MAX_POS = (ns[k] for k in ("L", "H", "D", "HQ", "NB", "MAX_POS"))
    store_k, store_v, q = drawn[0], drawn[1], drawn[2]
    new = drawn[3:]                                     # (k_new, v_new) per layer

    def raw(t):
        return gu.raw_view(t.contiguous().cpu()).reshape(-1)

    plane, block = 16 * D, 2 * H * 16 * D
    flat = np.zeros(L * NB * block, dtype=np.uint16)
    kp, vp = flat, flat[H * plane:]
    spec = PoolSpec(L, NB, H, D, "bf16", NB * block, block, plane)
    model = AllocatorModel(NB, 2, 32)
    model.alloc_blocks(0, 180)
    model.alloc_blocks(1, 100)
    o_cos, o_sin = rope_table(D, 10000.0, MAX_POS)
    lens = o_inject.inject(kp, vp, spec, model.tables, [0, 0], ns["runs"], raw(store_k),
                           raw(store_v), 300 * H * D, H * D, 0, L, "pairs", o_cos, o_sin)
    for s, n in enumerate(lens):
        model.set_len(s, n)
    model.extend([0, 1], 1)
    for layer in range(L):
        k_new = raw(new[2 * layer]).reshape(2, 1, H, D)
        v_new = raw(new[2 * layer + 1]).reshape(2, 1, H, D)
        o_inject.append(kp, vp, spec, layer, model.tables, model.lens, [0, 1], 1, k_new, v_new,
                        "pairs", o_cos, o_sin)
    gu.assert_bytes_equal(gu.raw_view(ns["buf"].cpu()), flat, "pool after the quick start")
    ref, ref_lse = o_att.decode_paged(raw(q).reshape(2, HQ, D), kp, vp, spec, L - 1,
                                      model.tables, model.lens, HQ)
    gu.assert_close(ns["out"].cpu().numpy(), ref, "out")
    gu.assert_close(ns["lse"].cpu().numpy(), ref_lse, "lse")
