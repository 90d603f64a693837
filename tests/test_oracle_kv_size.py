"""Pins the KV-size closed form against the figures the pages print."""
import json
import os

import pytest

from oracle.kv_size import kv_bytes, paged_pool_bytes
from tests.conftest import GOLDEN

UNITS = {"GB": 1e9, "MiB": 2 ** 20, "KiB": 2 ** 10, "GiB": 2 ** 30, "MB": 1e6}

with open(os.path.join(GOLDEN, "kv_size_printed.json")) as f:
    CASES = json.load(f)["cases"]


@pytest.mark.parametrize("case", CASES, ids=[c["cite"][:60] for c in CASES])
def test_printed_sizes(case):
    got = kv_bytes(case["L"], case["h"], case["d"], case["b"], case["n"])
    assert got == case["exact_bytes"]
    scaled = got / UNITS[case["unit"]]
    if "printed" in case:
        tol = case.get("printed_tolerance", 0.5 * 10 ** -(len(str(case["printed"]).split(".")[-1])
                                                         if "." in str(case["printed"]) else 0.5))
        assert abs(scaled - case["printed"]) <= tol, (scaled, case["printed"])
    if "printed_lower_bound" in case:
        assert scaled > case["printed_lower_bound"]


def test_linear_in_every_factor():
    base = kv_bytes(3, 5, 7, 2, 11)
    assert kv_bytes(6, 5, 7, 2, 11) == 2 * base
    assert kv_bytes(3, 10, 7, 2, 11) == 2 * base
    assert kv_bytes(3, 5, 14, 2, 11) == 2 * base
    assert kv_bytes(3, 5, 7, 4, 11) == 2 * base
    assert kv_bytes(3, 5, 7, 2, 22) == 2 * base
    assert kv_bytes(3, 5, 7, 2, 0) == 0


def test_gqa_divides_by_group():
    # Grouped-query example: 32 query heads in groups of four -> 8 KV heads,
    # four times less to store than with one KV head per query head.
    assert kv_bytes(32, 32, 128, 2, 1000) == 4 * kv_bytes(32, 8, 128, 2, 1000)


@pytest.mark.parametrize("n", [1, 15, 16, 17, 150, 8192])
def test_paged_waste_below_one_block(n):
    exact = kv_bytes(1, 1, 1, 1, n)
    paged = paged_pool_bytes(1, 1, 1, 1, n)
    assert 0 <= paged - exact <= 2 * 15
    assert paged % 32 == 0


def test_rejects_non_integers():
    with pytest.raises(ValueError):
        kv_bytes(1, 1, 1, 1, -1)
