"""Pins of the oracle's accounting functions to the pages' worked numbers."""
import json
import math
import os
from fractions import Fraction

import pytest

from conftest import GOLDEN
from oracle import accounting as acc

with open(os.path.join(GOLDEN, "accounting.json")) as f:
    GOLD = json.load(f)


@pytest.mark.parametrize("case", GOLD["bytes_per_token"], ids=lambda c: c["cite"][:40])
def test_bytes_per_token(case):
    L, H, d, b = case["L"], case["Hkv"], case["d"], case["b"]
    per = acc.kv_bytes_per_token(L, H, d, b)
    if "per_token" in case:
        assert per == case["per_token"]
    if "per_token_kib" in case:
        assert per == case["per_token_kib"] * 1024
    req = acc.kv_bytes(L, H, d, b, [case["tokens"]])
    assert req == case["request_gib"] * acc.GIB
    if "request_bytes" in case:
        assert req == case["request_bytes"]
    if "sequences" in case:
        batch = acc.kv_bytes(L, H, d, b, [case["tokens"]] * case["sequences"])
        assert batch == case["batch_bytes"]
        assert batch == case["batch_gib"] * acc.GIB


def test_ratios():
    for r in GOLD["ratios"]:
        if "base" not in r:
            assert r["Hq"] // r["Hkv"] == r["group"] and r["Hq"] % r["Hkv"] == 0
            # the stored cache is sized by KV heads, not query heads
            assert acc.kv_bytes_per_token(1, r["Hkv"], 128, 2) * 5 == acc.kv_bytes_per_token(1, r["Hq"], 128, 2)
            continue
        base = dict(r["base"])
        changed = dict(base, **r["change"])
        f = lambda c: acc.kv_bytes(c["L"], c["Hkv"], c["d"], c["b"], [c["tokens"]])
        assert f(changed) == r["factor"] * f(base)


def test_pages_for_500_tokens():
    c = GOLD["pages"][0]
    assert acc.blocks_for(c["T"], c["B"]) == c["blocks"]
    assert acc.allocated_slots(c["T"], c["B"]) == 512
    u = GOLD["pages"][2]
    assert abs(acc.paged_utilisation([u["T"]], u["B"]) - u["utilisation_about"]) <= u["abs_tol"]


def test_mean_tail_about_8_tokens():
    c = GOLD["pages"][1]
    m = acc.mean_tail_waste(c["B"], 512)
    assert m == Fraction(15, 2)
    assert abs(float(m) - c["mean_tail_about"]) <= c["abs_tol"]


def test_mean_tail_is_half_B_minus_one():
    c = GOLD["tail_waste"][0]
    for B in c["B"]:
        assert acc.mean_tail_waste(B, c["T_max"]) == Fraction(B - 1, 2), B
    # a page size that does not divide 512 breaks the identity (sanity of the test)
    assert acc.mean_tail_waste(3, 512) != Fraction(3 - 1, 2)


def test_reservation_waste_255_5():
    c = GOLD["tail_waste"][1]
    assert acc.mean_reservation_waste(c["reserve"], c["T_max"]) == Fraction(511, 2)
    assert float(acc.mean_reservation_waste(c["reserve"], c["T_max"])) == c["mean"]


def test_tail_range():
    for B in (1, 2, 5, 16, 64):
        for T in range(1, 300):
            w = acc.tail_waste(T, B)
            assert 0 <= w <= B - 1
            assert (T + w) % B == 0
    assert acc.blocks_for(0, 16) == 0


def test_utilisation():
    c = GOLD["utilisation"][0]
    u = acc.naive_utilisation(c["mean"], c["max"])
    assert 1 - u > c["unused_more_than"]
    c = GOLD["utilisation"][1]
    u = acc.naive_utilisation(c["mean"], c["max"])
    assert abs(u - c["naive_about"]) <= c["abs_tol"]
    paged = acc.paged_utilisation([c["mean"]], 16)
    assert abs(paged - c["paged_about"]) <= 0.005
    assert abs((paged - u) * 100 - c["gap_points_about"]) <= c["gap_tol"]


def test_decode_kv_bytes_matches_workload_sum():
    # one decode call over lengths reads the per-token cost times sum n
    lengths = [1, 7, 16, 33]
    assert acc.decode_kv_bytes(lengths, 1, 64, 4) == 2 * 1 * 64 * 4 * 57
    assert acc.decode_kv_bytes([32768] * 16, 8, 128, 2) == 2 ** 31
