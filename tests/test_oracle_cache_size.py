"""Pins for oracle.cache_size against the figures the pages print
(tests/golden/cache_size_figures.json, each entry cited)."""
import json
import math
import os

import pytest

from oracle import cache_size as cs

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "cache_size_figures.json")))


def test_mha_bytes_per_token():
    g = GOLD["mha_bytes_per_token_fp16"]
    elems = cs.mha_elems_per_token(g["heads"], g["d_head"], g["layers"])
    assert cs.cache_bytes(elems, 1, g["bytes_per_elem"]) == g["printed_kib"] * 1024


def test_values_per_token_table():
    g = GOLD["values_per_token_table"]
    # MHA with H * d_head = d_model: 2 * d_model values per token and layer
    mha = cs.mha_elems_per_token(1, g["d_model"])
    mla = cs.mla_elems_per_token(g["d_c"], g["d_rope"])
    assert mha == g["mha_values"] and mla == g["mla_values"]
    assert math.floor(10 * mha / mla) / 10 == g["ratio_printed"]
    gb = lambda e: cs.cache_bytes(e * g["layers"], g["tokens"], g["bytes_per_elem"]) / 1e9
    assert math.floor(10 * gb(mla)) / 10 == g["mla_gb_printed"]
    # the page rounds the MHA figure loosely (65.5 GB printed as 64 GB)
    assert gb(mha) == pytest.approx(g["mha_gb_printed"], rel=0.03)


def test_reduction_and_compute_factor():
    g = GOLD["reduction_at_d_c_512"]
    assert g["d_model"] / g["d_c"] == g["printed_ratio"]
    g = GOLD["naive_upprojection_factor"]
    assert 2 * g["d_c"] == g["printed"]


def test_toy_tutor():
    g = GOLD["toy_tutor"]
    b = cs.cache_bytes(cs.mha_elems_per_token(g["heads"], g["d_head"], g["layers"]),
                       g["tokens"], g["bytes_per_elem"])
    # the formula gives the product of the page's own factors, 2*4*4*16*32*4 ...
    assert b == 2 * 4 * 4 * 16 * 32 * 4 == 65536
    # ... which is twice the figure the page prints (a slip on the page)
    assert b == 2 * g["printed_kb"] * 1024
    assert round(g["printed_kb"] / g["reduction"], 1) == g["printed_reduced_kb"]


def test_gqa_equivalent_groups():
    g = GOLD["gqa_groups"]
    assert cs.gqa_groups_equivalent(g["d_c"], g["d_rope"], g["d_head"]) == g["printed_groups"]


def test_deepseek_v3_example():
    g = GOLD["deepseek_v3_example"]
    e = cs.mla_elems_per_token(g["kv_lora_rank"], g["qk_rope_head_dim"], g["num_hidden_layers"])
    assert e == g["printed_elems_per_token"]
    assert cs.cache_bytes(e, g["context"], g["bytes_per_elem"]) / 2 ** 30 == g["printed_gib"]


def test_table9_with_inferred_shapes():
    g = GOLD["table9"]
    for key, (layers, nhdh) in {"small_moe": (27, 2048), "large_moe": (60, 7168)}.items():
        mla = cs.mla_elems_per_token(512, 64, layers)
        mha = cs.mha_elems_per_token(1, nhdh, layers)
        assert round(mla / 1000, 1) == g[key]["mla_printed_k"]
        assert round(mha / 1000, 1) == g[key]["mha_printed_k"]


def test_mla_formula_is_not_mha_formula():
    # a dropped factor of 2 or a per-head latent would break these
    assert cs.mha_elems_per_token(128, 128, 1) == 32768
    assert cs.mla_elems_per_token(512, 64, 1) * 128 != cs.mla_elems_per_token(512, 64, 128) * 2
