"""Pins for oracle/accounting.py against the numbers the pages print
(tests/golden/pages_numbers.json carries each number with its source)."""

import json
import os

from oracle import accounting as acc
from oracle import layout

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_numbers.json")))


def g(k):
    return GOLD[k]["value"]


def test_page_and_buffer_sizes():
    assert g("c4r4_page_bytes") == acc.PAPER_C4R4_PAGE
    assert g("c4r4_page_bytes") // 64 == g("c4r4_bytes_per_token")
    assert acc.PROT_BYTES == g("prot_bytes_per_request_layer")
    assert acc.BF16_PAGE == g("bf16_page_bytes")
    assert acc.REVERSE_MAP_BYTES == g("reverse_map_bytes_per_page")
    assert layout.PROT_ROWS == g("sink_tokens") + g("recent_tokens")


def test_compression_ratios_printed():
    for k in ("compression_4k", "compression_128k"):
        e = GOLD[k]
        assert round(acc.compression(e["L"]), e["digits"]) == e["value"]


def test_compression_with_library_page():
    # this library's pages carry bf16 scale+zero for all 9 groups
    assert round(acc.compression(4096, layout.page_bytes("C4R4")), 2) == 3.19
    assert round(acc.compression(131072, layout.page_bytes("C4R4")), 2) == 3.54


def test_compression_with_fp32_rope_metadata_page():
    # C4R4F: 20,992-byte pages (328 B/token against the pages' 320); by hand,
    # 4K: 64 * 73,728 / (64 * 21,000 + 152,064) = 4,718,592 / 1,496,064
    # 128K: 2048 * 73,728 / (2048 * 21,000 + 152,064) = 150,994,944 / 43,160,064
    assert layout.page_bytes("C4R4F") == 20992
    assert acc.packed_bytes(4096, 20992) == 1496064
    assert acc.packed_bytes(131072, 20992) == 43160064
    assert round(acc.compression(4096, 20992), 2) == 3.15
    assert round(acc.compression(131072, 20992), 2) == 3.50


def test_schema_counts():
    e = GOLD["mha_elements_per_token_layer"]
    assert acc.mha_elements(e["heads"], e["head_dim"]) == e["value"]
    e2 = GOLD["mla_elements_per_token_layer"]
    assert acc.mla_elements(e2["d_c"], e2["d_r"]) == e2["value"]
    assert round(e["value"] / e2["value"], 1) == g("mha_over_mla_ratio")


def test_cache_sizes_60_layers_128000_tokens():
    e = GOLD["mla_cache_gb_60L_128000tok"]
    b = acc.mla_cache_bytes(e["layers"], e["tokens"], e["batch"], 512, 64, e["bytes_per_elem"])
    assert round(acc.gb(b), 2) == e["value"]
    assert round(acc.gib(b), 2) == g("mla_cache_gib_60L_128000tok")
    bm = acc.mha_cache_bytes(e["layers"], e["tokens"], e["batch"], 128, 128, 2)
    assert round(acc.gib(bm), 1) == g("mha_cache_gib_60L_128000tok")


def test_serving_budget_exceeds_bf16_slots():
    e = GOLD["serving_requests"]
    total = e["value"] * (e["input_tokens"] + e["output_tokens"])
    assert total == g("serving_token_budget")
    assert total > g("serving_bf16_usable_slots")
