"""The pages' printed numbers (tests/golden/pages_numbers.json) against the
byte accounting of the three-segment INT2 pool."""

import json
import os

from synthetic import CONFIGS

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_numbers.json")))


def _g(name):
    return GOLD[name]["value"]


def test_history_bits_per_element_is_2_25():
    wl = CONFIGS["qwen3-8b-l100k"]
    # 2 bits per code + a bf16 scale and zero per 128-channel group
    bits = wl.int2_bytes_per_token_head() * 8 / (2 * wl.head_dim)
    assert bits == _g("int2_baseline_bits_per_element") == 2 + 32 / _g("group_size_launch")


def test_overall_bits_per_element_is_2_28_at_128k():
    L = 131_072
    bf16 = _g("sink_tokens") + _g("recent_tokens")
    bpe = (bf16 * 16 + (L - bf16) * 2.25) / L
    assert round(bpe, 2) == _g("bits_per_kv_element")
    assert round(100 * bf16 / L, 2) == _g("bf16_share_at_128k_percent")
    assert round(16 / bpe) == _g("kv_memory_reduction_overall")
    assert 16 / 2 == _g("kv_memory_reduction_history")


def test_four_codes_per_byte_four_levels():
    assert 8 // 2 == _g("codes_per_byte") and 2 ** 2 == _g("int2_levels")


def test_headline_workload_byte_counts():
    kv = CONFIGS["qwen3-8b-l100k"].kv_bytes()
    assert kv["int2"] == 57_415_680 and kv["bf16"] == 1_310_720
    assert kv["bf16_only_total"] == 409_600_000
    kv2 = CONFIGS["qwen3-8b-b32-l32k-demote"].kv_bytes()
    assert kv2["int2"] == 598_081_536 and kv2["bf16"] == 41_943_040
