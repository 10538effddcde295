"""The workload presets against the numbers the pages fix (tests/golden/pages_defaults.json)."""
import json
import os

from kv_cache_eviction_continual_amd import configs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_presets_use_the_published_defaults():
    g = json.load(open(os.path.join(GOLDEN, "pages_defaults.json")))
    for cfg in (2, 3, 4):
        w = configs.get(cfg)
        assert (w.n_recent, w.n_beacons, w.window) == (g["n_recent"], g["n_beacons"], g["window"])


def test_qwen3_4b_shape_reproduces_the_77GB_cache():
    g = json.load(open(os.path.join(GOLDEN, "pages_defaults.json")))
    w = configs.get(3)
    q = g["qwen3_4b"]
    assert (w.layers, w.n_kv_heads, w.head_dim) == (q["layers"], q["kv_heads"], q["head_dim"])
    per_token = w.layers * w.n_kv_heads * w.head_dim * 2 * q["bytes_per_elem"]  # K and V
    assert per_token == 147456
    assert round(per_token * 16 * 32768 / 1e9) == g["kv_gb_batch16_32k"]


def test_throughput_table_is_batch_times_32k_over_latency():
    g = json.load(open(os.path.join(GOLDEN, "pages_defaults.json")))
    # the printed latencies are whole seconds, so agreement is to ~0.1 %
    assert abs(g["batch"] * 32768 / g["latency_full_s"] / g["full_kv_tok_s"] - 1) < 1e-3
    assert abs(g["batch"] * 32768 / g["latency_beaconkv_s"] / g["beaconkv_tok_s"] - 1) < 1e-3
