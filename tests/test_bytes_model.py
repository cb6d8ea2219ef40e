"""The byte model against the numbers the pages print (tests/golden/pages_byte_model.json)."""
import json
import os

from nvfp4_bit_projection_amd import bytes_model as bm

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_byte_model.json")))
S = bm.LayerShape()
V = 150144


def test_parameter_counts():
    L = GOLD["moe_layers"]
    routed_total = L * S.n_experts * 3 * S.expert_width * S.hidden
    assert round(routed_total / 1e9, 2) == GOLD["routed_params_total_billions_printed"]
    routed_read = L * S.top_k * 3 * S.expert_width * S.hidden
    assert round(routed_read / 1e6) == GOLD["routed_params_read_per_token_millions_printed"]
    assert round(V * S.hidden / 1e6, 1) == GOLD["head_params_millions_printed"]


def test_bits_and_head_row():
    assert 8 * bm.nvfp4_bytes(1, 2048) / 2048 == GOLD["bits_per_weight_printed"]
    assert 2048 // 2 == GOLD["head_row_code_bytes_printed"]


def test_megabytes_per_token():
    L = GOLD["moe_layers"]
    assert round(L * S.top_k * bm.expert_bytes(S) / 1e6) == GOLD["routed_mb_per_token_printed"]
    assert round(bm.head_bytes(V, S.hidden) / 1e6) == GOLD["head_mb_per_token_printed"]


def test_stack_totals():
    assert bm.layer_bytes(S) == 16_252_928
    assert bm.head_bytes(V, 2048) == 172_965_888
    assert bm.token_bytes(S, 47, V) == 936_853_504
    assert bm.layer_bytes(bm.LayerShape(n_experts=32)) == 14_417_920
    assert abs(bm.expected_distinct_experts(256, 6, 8) - 44.24) < 0.01
