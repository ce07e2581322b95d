"""Oracle pins: KV-cache size formulas against the numbers the pages print.

Page keys as in tests/golden/page_numbers.json (LC, PA, SO).
"""
import json
import os

import pytest

from oracle import sizes

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_numbers.json")))


def test_llama3_bytes_per_token():
    # LC opening formula: 2 x 32 layers x 8 KV heads x 128 x 2 bytes
    assert sizes.kv_bytes_per_token(32, 8, 128, 2) == GOLD["llama3_8b_bytes_per_token"]["value"]


def test_llama3_128k_tokens_about_16gb():
    g = GOLD["llama3_8b_128k_tokens_gb"]
    b = sizes.kv_cache_bytes(32, 8, 128, g["tokens"])
    # "about 16 GB": 16.78e9 bytes = 15.6 GiB; both readings round to 16
    assert abs(b / 1e9 - g["value"]) < 1.0 and abs(b / sizes.GIB - g["value"]) < 0.5


def test_kv_cache_gb_printed_values_are_twice_the_formula():
    g = GOLD["kv_cache_gb_printed"]
    for call, printed in zip(g["calls"], g["values"]):
        n_layers, n_kv, hd, max_len, batch, dtb = call
        formula = sizes.kv_cache_gib(n_layers, n_kv, hd, max_len, batch, dtb)
        # the function the page defines returns half of what it prints next to it
        assert formula * 2 == printed
        assert sizes.kv_cache_gib(n_layers, n_kv, hd, max_len, batch, 2 * dtb) == printed


def test_formula_agrees_with_section5_per_request_sizes():
    g = GOLD["so_128k_per_request_gb"]
    assert sizes.kv_cache_gib(32, 8, 128, 131072, dtype_bytes=1) == g["fp8"]
    assert sizes.kv_cache_gib(32, 8, 128, 131072, dtype_bytes=2) == g["fp16"]
    assert sizes.kv_cache_gib(32, 8, 128, 8192, dtype_bytes=2) == g["window_8k_fp16"]


def test_llama2_70b_table():
    g = GOLD["llama2_70b_gib"]
    exact = [sizes.kv_cache_bytes(80, 8, 128, s) / sizes.GIB for s in g["seq_lens"]]
    assert exact == [0.625, 2.5, 10.0]
    for e, p in zip(exact, g["printed"]):
        assert abs(e - p) <= 0.005 + 1e-12          # page rounds 0.625 up to 0.63
    assert 8 * sizes.kv_cache_bytes(80, 8, 128, 32768) / sizes.GIB == GOLD["llama2_70b_batch8_32k_gib"]["value"]
    fp16, int8 = GOLD["llama2_70b_32k_fp16_int8_gib"]["values"]
    assert sizes.kv_cache_bytes(80, 8, 128, 32768, 2) / sizes.GIB == fp16
    assert sizes.kv_cache_bytes(80, 8, 128, 32768, 1) / sizes.GIB == int8


@pytest.mark.parametrize("name", ["A", "B", "C"])
def test_blocks_and_last_fill(name):
    r = GOLD["pa_layout_example"]["requests"][name]
    assert sizes.blocks_needed(r["tokens"]) == len(r["blocks"])
    assert sizes.last_block_fill(r["tokens"]) == r["last_fill"]


def test_blocks_needed_edges():
    assert [sizes.blocks_needed(n) for n in (0, 1, 15, 16, 17, 32, 33)] == [0, 1, 1, 1, 2, 2, 3]
    assert [sizes.last_block_fill(n) for n in (0, 1, 16, 17)] == [0, 1, 16, 1]
