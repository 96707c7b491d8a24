"""Pins of the oracle's byte accounting to the byte counts the pages print
(tests/golden/page_numbers.json lists each figure and where it is printed)."""
import json
import os

import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden", "page_numbers.json")
ITEMS = json.load(open(GOLD))["items"]


def _bytes(it):
    sh = it["shape"]
    if it["kind"] == "call_bytes":
        return oracle.algorithmic_bytes(sh["M"], sh["V"], sh["K"], sh["bits"], sh["group"])
    if it["kind"] == "dense_weight_bytes":
        return sh["V"] * sh["K"] * sh["bytes_per_weight"]
    if it["kind"] == "freed":
        packed = oracle.packed_bytes(sh["V"], sh["K"], sh["bits"], sh["group"])
        return sh["V"] * sh["K"] * sh["dense_bytes_per_weight"] - packed
    raise AssertionError(it["kind"])


@pytest.mark.parametrize("it", ITEMS, ids=[i["id"] for i in ITEMS])
def test_page_byte_counts(it):
    got = _bytes(it) / it["unit"]
    assert abs(got - it["value"]) <= it["tol"], (it["printed"], got)


def test_packed_bytes_equal_weight_plus_scales_when_rows_fill_blocks():
    # 248064, 151936 and 50304 are multiples of the 64-row block: no padding bytes
    for V, K, b, G in [(248064, 5120, 4, 128), (151936, 1024, 4, 64), (151936, 1024, 8, 128),
                       (151936, 2048, 8, 2048), (50304, 512, 4, 64)]:
        assert oracle.packed_bytes(V, K, b, G) == V * K * b // 8 + V * (K // G) * 2
