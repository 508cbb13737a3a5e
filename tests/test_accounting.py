"""Byte accounting and arithmetic intensity against the figures the pages print
(tests/golden/page_figures.json; each entry carries its page and section)."""
import json
import os

import numpy as np
import pytest

from oracle import accounting as acc

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.json"), encoding="utf-8"))


def test_pin_b_active_bytes_26_tokens():
    g = GOLD["v2lite_active_26_tokens"]
    n = acc.naive_cache_bytes(g["tokens"], heads=g["heads"])
    a = acc.absorbed_cache_bytes(g["tokens"])
    assert n == g["naive_total_bytes"] == g["naive_key_bytes"] + g["naive_value_bytes"]
    assert a == g["absorb_total_bytes"] == g["absorb_latent_bytes"] + g["absorb_rope_bytes"]
    assert acc.naive_cache_bytes(g["tokens"], heads=16, v_head=0) == g["naive_key_bytes"]
    assert acc.absorbed_cache_bytes(g["tokens"], d_r=0) == g["absorb_latent_bytes"]
    assert str(n / a).startswith(g["ratio_text"])       # the page truncates: 8.888888...
    assert n * 9 == a * 80                         # 8.888... = 80/9 exactly
    assert 100 * (1 - a / n) == pytest.approx(g["reduction_percent"], abs=1e-12)


def test_allocated_32_slot_bytes():
    g = GOLD["v2lite_allocated_32_slots"]
    assert acc.naive_cache_bytes(g["slots"], heads=16) == g["naive_total_bytes"]
    assert acc.naive_cache_bytes(g["slots"], heads=16, v_head=0) == g["naive_key_bytes"]
    assert acc.absorbed_cache_bytes(g["slots"]) == g["absorb_total_bytes"]
    assert acc.absorbed_cache_bytes(g["slots"], d_r=0) == g["absorb_latent_bytes"]


def test_pin_c_1152_bytes_per_token():
    g = GOLD["v2lite_elements_per_token"]
    assert acc.absorbed_cache_bytes(1) == 1152 == 2 * g["absorbed_elements"]
    assert acc.naive_cache_bytes(1, heads=16) == 2 * g["naive_elements"]
    assert acc.naive_cache_bytes(1, heads=16, v_head=0) == 2 * g["key_elements"]


def test_v3_per_token_table():
    g = GOLD["v3_per_token_table"]
    assert acc.per_token_elements("mha") == g["mha_elements"]
    assert acc.per_token_elements("gqa", kv_heads=8) == g["gqa8_elements"]
    assert acc.per_token_elements("mqa") == g["mqa_elements"]
    assert acc.per_token_elements("mla") == g["mla_elements"]
    for k in ("mha", "gqa8", "mqa", "mla"):
        assert g[k + "_bytes"] == 2 * g[k + "_elements"]
    assert round(g["mha_elements"] / g["mla_elements"]) == g["mha_over_mla_approx"]
    assert round(100 * (1 - g["mla_elements"] / g["mha_elements"]), 1) == g["reduction_percent_1dp"]
    assert round(g["layers"] * acc.absorbed_cache_bytes(1) / 1000) == g["all_layers_kb_approx"]


def test_v2_vs_67b_decomposition():
    g = GOLD["v2_vs_67b"]
    b67 = 2 * g["b67_kv_heads"] * 128 * 2 * g["b67_layers"] / 1024
    assert round(b67) == g["b67_kb_per_token_approx"]
    v2 = 60 * acc.absorbed_cache_bytes(1) / 1024            # V2: 60 layers
    assert v2 == g["v2_bf16_kb_per_token"]
    assert round(100 * (1 - v2 / b67), 1) == g["same_precision_reduction_percent"]
    v2q = v2 * 6 / 16
    assert round(v2q, 1) == g["v2_6bit_kb_per_token"]
    assert round(100 * (1 - v2q / b67), 1) == g["headline_reduction_percent"]
    assert acc.per_token_elements("mla") / (2 * 128) == g["mla_as_gqa_groups"]


def test_report_sizes_scale_free():
    g = GOLD["report_per_token_sizes"]
    L = g["layers"]
    assert acc.naive_cache_bytes(1, heads=16) == g["expanded_bytes_per_layer"]
    full = g["expanded_bytes_per_layer"] * L / 1024
    assert round(full) == g["expanded_kb"]
    ab = acc.absorbed_cache_bytes(1) * L / 1024
    i8 = acc.absorbed_cache_bytes(1, elem_bytes=1) * L / 1024
    i4 = acc.absorbed_cache_bytes(1) * L / 4 / 1024              # 4 bits an element
    assert round(ab, 1) == g["absorbed_kb"] and round(full / ab, 1) == g["absorbed_ratio"]
    assert round(i8, 1) == g["int8_kb"] and round(full / i8, 1) == g["int8_ratio"]
    assert round(i4, 1) == g["int4_kb"] and round(full / i4, 1) == g["int4_ratio"]
    assert round(10 * 2 ** 30 / (i8 * 1024) / 1e4) == g["int8_tokens_in_10gb_wan"]
    assert round(10 * 2 ** 30 / (i4 * 1024) / 1e4) == g["int4_tokens_in_10gb_wan"]


def _count_decode_flops_and_bytes(H, L, d_c=512, d_r=64, elem=2):
    """Count the multiply-adds of one absorbed decode step by walking the two
    contractions (scores over 576 = d_c + d_r, weighted sum over d_c) token by
    token; bytes are the cached elements read once."""
    flops = 0
    for _t in range(L):
        for _h in range(H):
            flops += 2 * (d_c + d_r)          # score: one multiply-add per width element
            flops += 2 * d_c                  # value: one multiply-add per latent element
    return flops, L * (d_c + d_r) * elem


@pytest.mark.parametrize("H", [16, 128])
def test_decode_ai_matches_counted_work(H):
    f, b = _count_decode_flops_and_bytes(H, 3)
    assert acc.decode_ai("mla", H) == pytest.approx(f / b, rel=1e-15)
    assert f / 3 == 2176 * H


def test_ridge_heads_and_mha_ai():
    # MHA/GQA AI does not depend on sequence length: 2 H_q / (H_kv b)
    assert acc.decode_ai("mha", 128, 128) == 1.0
    assert acc.decode_ai("gqa", 128, 8) == 16.0
    h = acc.heads_to_cross_ridge(1000e12 / 3e12)
    assert acc.decode_ai("mla", h) == pytest.approx(1000 / 3, rel=1e-12)
    assert 128 < h < 256           # V3's 128 heads sit below that balance point


def test_tilelang_budget_conclusions():
    g = GOLD["budget_part_c"]
    o, s, tot = acc.tilelang_register_budget(g["block_h"], g["block_n"], 512, g["threads"])
    assert tot <= g["register_limit"] and (tot <= 255) == g["fits_registers"]
    smem = acc.tilelang_smem_sum(g["block_h"], g["block_n"], 512, 64, g["stages"])
    assert (smem > g["h100_smem_kb"] * 1024) == g["exceeds_h100_smem"]
    assert o == g["block_h"] * 512 / g["threads"]
