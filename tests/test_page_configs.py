"""Layer resolution pinned to the configuration tables and ratios the pages print."""
import json
import os

import pytest

from oracle import gemma_ref as R

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_configs.json")))


@pytest.mark.parametrize("ratio", GOLDEN["ratios"], ids=lambda r: f"pattern{r['pattern']}")
def test_local_global_ratio(ratio):
    cfg = R.GemmaAttnConfig(num_heads=8, num_kv_heads=1, head_dim=64, sliding_window=512,
                            sliding_window_pattern=ratio["pattern"])
    period = ratio["local"] + ratio["global"]
    for start in range(0, 4 * period, period):
        kinds = [R.resolve_layer(cfg, layer)["is_global"] for layer in range(start, start + period)]
        assert kinds.count(False) == ratio["local"] and kinds.count(True) == ratio["global"]


def test_gemma4_table_layers():
    m = GOLDEN["models"]["gemma4"]
    bases = GOLDEN["rope_bases"]
    cfg = R.GemmaAttnConfig(num_heads=m["num_heads"], num_kv_heads=m["num_kv_heads"], head_dim=m["head_dim"],
                            num_global_kv_heads=m["num_global_kv_heads"], global_head_dim=m["global_head_dim"],
                            sliding_window=m["sliding_window"], sliding_window_pattern=m["sliding_window_pattern"],
                            rope_theta=bases["global"], rope_local_theta=bases["local"],
                            partial_rotary_factor=m["partial_rotary_factor"], k_eq_v=m["k_eq_v"])
    layers = [R.resolve_layer(cfg, i) for i in range(m["num_layers"])]
    assert sum(L["is_global"] for L in layers) == m["num_layers"] // m["sliding_window_pattern"]
    g = [L for L in layers if L["is_global"]][0]
    loc = [L for L in layers if not L["is_global"]][0]
    assert (g["num_kv_heads"], g["head_dim"], g["k_eq_v"], g["window"], g["theta"]) == (1, 512, True, 0, 1e6)
    assert (loc["num_kv_heads"], loc["head_dim"], loc["k_eq_v"], loc["window"], loc["theta"]) == (8, 256, False, 1024, 1e4)
    assert g["rotary_dim"] == 128 and loc["rotary_dim"] == 64     # a quarter of each head rotated
    assert g["group"] == 16 and loc["group"] == 2


def test_gemma2_alternating_and_gemma3_stack():
    m2 = GOLDEN["models"]["gemma2"]
    cfg2 = R.GemmaAttnConfig(num_heads=m2["num_heads"], num_kv_heads=m2["num_kv_heads"], head_dim=m2["head_dim"],
                             sliding_window=m2["sliding_window"], sliding_window_pattern=m2["sliding_window_pattern_reading"],
                             query_pre_attn_scalar=m2["query_pre_attn_scalar"],
                             attn_logit_softcapping=m2["attn_logit_softcapping"])
    kinds = [R.resolve_layer(cfg2, i)["is_global"] for i in range(m2["num_layers"])]
    assert kinds == [i % 2 == 1 for i in range(m2["num_layers"])]
    L = R.resolve_layer(cfg2, 0)
    assert L["scale"] == 256.0 ** -0.5 and L["softcap"] == 50.0 and L["group"] == 2
    m3 = GOLDEN["models"]["gemma3"]
    cfg3 = R.GemmaAttnConfig(num_heads=m3["num_heads"], num_kv_heads=m3["num_kv_heads"], head_dim=m3["head_dim"],
                             sliding_window=m3["sliding_window"], sliding_window_pattern=m3["sliding_window_pattern"],
                             rope_theta=m3["rope_theta"], rope_local_theta=m3["rope_local_theta"])
    thetas = [R.resolve_layer(cfg3, i)["theta"] for i in range(6)]
    assert thetas == [1e4] * 5 + [1e6]
    assert sum(R.resolve_layer(cfg3, i)["is_global"] for i in range(m3["num_layers"])) == m3["num_layers"] // 6


def test_window_disabled_means_all_global():
    m = GOLDEN["models"]["gemma"]
    cfg = R.GemmaAttnConfig(num_heads=m["num_heads"], num_kv_heads=m["num_kv_heads"], head_dim=m["head_dim"],
                            sliding_window=0, sliding_window_pattern=6)
    assert all(R.resolve_layer(cfg, i)["is_global"] for i in range(m["num_layers"]))
    assert R.resolve_layer(cfg, 0)["group"] == 8          # multi-query: one KV head
