"""The byte/FLOP formulas the benchmark uses reproduce the derived figures
printed in the book's cost-model chapter (tests/golden/cost_model.json)."""

import json
import os

from sparse_attention_csa_amd import accounting as acc

G = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "cost_model.json")))


def test_cache_bytes():
    assert acc.gqa_bytes_per_token_layer() == G["gqa8_bf16_bytes_per_token_layer"]
    per_layer = acc.gqa_bytes_per_token_layer() * 10 ** 6
    assert per_layer / 1e9 == G["gqa8_gb_per_layer_at_1e6"]
    assert abs(per_layer * 61 / 1e9 - G["gqa8_gb_61_layers"]) < 1e-9
    assert abs(per_layer * 43 / 1e9 - G["gqa8_gb_43_layers"]) < 1e-9
    assert acc.mixed_entry_bytes() == G["entry_bytes_fp8_448_bf16_64"]
    assert acc.main_bytes_per_token(4) == G["csa_main_bytes_per_token"]
    assert acc.main_bytes_per_token(128) == G["hca_main_bytes_per_token"]
    assert acc.fp4_indexer_bytes_per_token() == G["fp4_indexer_bytes_per_token"]
    assert acc.csa_bytes_per_token() == G["csa_total_bytes_per_token"]
    assert round(acc.model_cache_bytes(10 ** 6, 30, 31) / 1e9, 2) == G["pro_model_gb_at_1e6"]
    assert round(acc.model_cache_bytes(10 ** 6, 21, 20) / 1e9, 2) == G["flash_model_gb_at_1e6"]


def test_flops():
    assert round(acc.attention_flops_per_query(512, 1024 + 128, 128) / 1e6) == \
        G["pro_csa_main_mflop_per_query_layer"]
    assert round(acc.attention_flops_per_query(512, 7812 + 128, 128) / 1e9, 2) == \
        G["pro_hca_main_gflop_per_query_layer"]
    assert acc.indexer_flops_per_query(64, 128, 10 ** 6) / 1e9 == G["indexer_gflop_per_query_layer"]
