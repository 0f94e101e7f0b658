"""Pins for oracle.accounting against the figures the page prints
(tests/golden/page_figures.json, each entry with its citation)."""

import json
import os

import oracle as O

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")))


def test_default_operating_point_is_2_26_bits():
    g = GOLD["default_config"]
    bpe = O.bits_per_elem(g["container_bytes_k"], g["container_bytes_v"],
                          g["group_values"], g["bf16_window_tokens"])
    assert round(bpe, 2) == g["bits_per_value"]


def test_key_value_split_2_68_and_1_84():
    g = GOLD["default_config"]
    n, W = g["group_values"], g["bf16_window_tokens"]
    k_bits = 8.0 * (g["container_bytes_k"] + 4 + (n + 2) / W) / n
    v_bits = 8.0 * (g["container_bytes_v"] + 4) / n
    assert round(k_bits, 2) == GOLD["kv_split"]["bits_k"]
    assert round(v_bits, 2) == GOLD["kv_split"]["bits_v"]
    # the split and the total are the same accounting
    assert abs((k_bits + v_bits) / 2 - O.bits_per_elem(331, 231, n, W)) < 1e-12


def test_metadata_convention_matches_int2_example():
    g = GOLD["fixed_width_example"]
    bits = (g["bits"] * g["group"] + 8 * g["metadata_bytes"]) / g["group"]
    assert bits == g["bits_per_value"]


def test_budget_helper():
    assert O.containers_for_budget(2.26, 1024, 128) == (331, 231)
    assert O.containers_for_budget(2.0, 1024, 128) == (292, 203)
    assert O.containers_for_budget(3.0, 1024, 128) == (442, 309)
    assert O.containers_for_budget(4.0, 1024, 128) == (593, 414)
    for b in (2.0, 2.26, 3.0, 4.0):
        ck, cv = O.containers_for_budget(b, 1024, 128)
        assert O.bits_per_elem(ck, cv, 1024, 128) <= b
    assert O.bits_per_elem(36, 36, 128, 128, metadata=False) == 2.25
