"""Pins of the byte accounting against the numbers the pages print."""
import json
import os
from fractions import Fraction

import pytest

from oracle import accounting as acc

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_numbers.json")))

MIB = 2 ** 20
GIB = 2 ** 30


def test_entry_costs_match_page_equations():
    assert acc.entry_bytes(512, 16) == GOLD["main_entry_bytes"]["value"]
    assert acc.entry_bytes(512, 0) == GOLD["main_entry_data_bytes"]["value"]
    assert acc.entry_bytes(512, 16) - acc.entry_bytes(512, 0) == GOLD["main_entry_scale_bytes"]["value"]
    assert acc.entry_bytes(128, 32) == GOLD["indexer_entry_bytes"]["value"]
    assert acc.entry_bytes(128, 0) == GOLD["indexer_entry_data_bytes"]["value"]
    assert acc.entry_bytes(128, 32) - acc.entry_bytes(128, 0) == GOLD["indexer_entry_scale_bytes"]["value"]


def test_per_layer_table_and_total():
    t = GOLD["per_layer_table"]
    main_sum = idx_sum = tot = Fraction(0)
    for row in t["rows"]:
        main = acc.entry_bytes(512, 16) / row["ratio"]
        idx = acc.entry_bytes(128, 32) / row["ratio"]
        assert main == Fraction(row["main"]).limit_denominator()
        assert idx == Fraction(row["indexer"]).limit_denominator()
        assert acc.layer_bytes_per_token(row["ratio"]) == Fraction(row["total"]).limit_denominator()
        main_sum += main
        idx_sum += idx
        tot += acc.layer_bytes_per_token(row["ratio"])
    assert main_sum == t["totals"]["main"]
    assert idx_sum == t["totals"]["indexer"]
    assert tot == t["totals"]["total"]
    ratios = [r["ratio"] for r in t["rows"]]
    assert acc.bytes_per_token(ratios) == GOLD["per_token_equation"]["total"]
    eq = GOLD["per_token_equation"]["terms"]
    assert acc.bytes_per_token([2, 2, 2]) == eq[0] and acc.bytes_per_token([1]) == eq[1]


@pytest.mark.parametrize("row", GOLD["context_table"]["rows"])
def test_context_table(row):
    per_token = acc.bytes_per_token([2, 2, 2, 1])
    total = acc.cache_bytes(row["tokens"], per_token)
    unit = MIB if row["unit"] == "MiB" else GIB
    assert round(float(total) / unit, row["digits"]) == row["printed"]


def test_v1_and_ratios():
    v1 = GOLD["v1_bytes_per_token"]
    b = acc.gqa_bf16_bytes_per_token(v1["layers"], v1["kv_heads"], v1["head_dim"], v1["elem_bytes"])
    assert b == v1["value"]
    assert round(b / float(acc.bytes_per_token([2, 2, 2, 1])), 1) == GOLD["v1_ratio"]["value"]
    v4 = GOLD["v4flash_bytes_per_token"]
    assert round(v4["value"] / float(acc.bytes_per_token([2, 2, 2, 1])), 2) == v4["ratio_printed"]


def test_sliding_window():
    s = GOLD["sliding_window"]
    b = acc.sliding_window_bytes(s["layers"], s["window"], s["channels"], s["block"])
    assert round(b / MIB, 2) == s["printed_mib"]
    glob = acc.cache_bytes(2 ** 20, acc.bytes_per_token([2, 2, 2, 1]))
    assert round(100 * b / float(glob), 1) == s["percent_of_global_at_1m"]


def test_counterfactuals_follow_the_formula_not_the_printed_numbers():
    c = GOLD["counterfactuals"]
    block32 = acc.bytes_per_token([2, 2, 2, 1], lat=(512, 32, 1), idx=(128, 32, 1))
    no_scales = acc.bytes_per_token([2, 2, 2, 1], lat=(512, 0, 1), idx=(128, 0, 1))
    assert block32 == 850 and no_scales == 800
    # the page's printed values are a known inconsistency, kept visible here
    assert (c["printed_block32_everywhere"], c["printed_without_scales"]) != (block32, no_scales)
