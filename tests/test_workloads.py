"""Seeded input generator: presets match the pages, calibration constants
match their recorded fit, generation is deterministic, bfloat16 rounding is
round-to-nearest-even, and the tie / hot-expert structures are as stated."""
import json
import os

import numpy as np

from sigmoid_group_limited_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_presets_match_pages():
    with open(os.path.join(GOLDEN, "model_presets.json")) as f:
        g = json.load(f)
    ds, km = g["deepseek_v3_671b"], g["kimi_k2"]
    assert (wl.DSV3.n_experts, wl.DSV3.n_group, wl.DSV3.topk_group, wl.DSV3.top_k,
            wl.DSV3.route_scale) == (ds["n_routed_experts"], ds["n_expert_groups"],
                                     ds["n_limited_groups"], ds["n_activated_experts"],
                                     ds["route_scale"])
    assert (wl.KIMI_K2.n_experts, wl.KIMI_K2.n_group, wl.KIMI_K2.top_k,
            wl.KIMI_K2.route_scale) == (km["n_routed_experts"], km["n_group"],
                                        km["top_k"], km["route_scale"])
    assert wl.D_MODEL == km["hidden_size"]


def test_calibration_constants_recorded():
    with open(os.path.join(GOLDEN, "workload_calibration.json")) as f:
        c = json.load(f)
    assert wl.TIE_PAIRS == c["tie_pairs"]
    assert wl.HOT_SHIFT == c["hot_shift"]
    assert abs(c["hot_share"] - 0.5) <= 0.01
    assert 0.005 <= c["tie_decisive_fraction"][str(c["tie_pairs"])] <= 0.02


def test_bf16_round_to_nearest_even():
    vals = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, -2.5, 1.0 + 2**-8 + 2**-20,
                     3.0e38, 1e-40], dtype=np.float32)
    bits = wl.bf16_bits(vals)
    assert bits[0] == 0x3F80
    assert bits[1] == 0x3F80          # halfway, ties to even (down)
    assert bits[2] == 0x3F82          # halfway, ties to even (up)
    assert bits[3] == 0xC020
    assert bits[4] == 0x3F81          # above halfway rounds up
    back = wl.bf16_to_f32(bits)
    assert back[0] == 1.0 and back[3] == -2.5
    assert np.all(np.abs(back[:5] - vals[:5]) <= np.abs(vals[:5]) * 2**-8)


def test_deterministic_and_shapes():
    a = wl.workload_inputs("dsv3-tiny")
    b = wl.workload_inputs("dsv3-tiny")
    assert a.x.shape == (64, 7168) and a.x.dtype == np.uint16
    assert a.W.shape == (256, 7168) and a.W.dtype == np.float32
    assert a.bias.shape == (256,) and a.bias.dtype == np.float32
    assert np.array_equal(a.x, b.x) and np.array_equal(a.W, b.W)
    assert np.array_equal(a.bias, b.bias)
    assert np.all(np.abs(a.bias) <= 0.05)
    assert abs(float(a.W.std()) * np.sqrt(7168) - 1.0) < 0.01


def test_twins_and_hot_experts():
    t = wl.workload_inputs("dsv3-prefill-ties", T=8)
    assert len(t.twins) == wl.TIE_PAIRS
    S = 256 // 8
    for a, b in t.twins:
        assert a // S == b // S and a != b
        assert np.array_equal(t.W[a], t.W[b]) and t.bias[a] == t.bias[b]
    h = wl.workload_inputs("dsv3-skewed", T=8)
    assert len(h.hot) == 16
    assert np.array_equal(np.bincount(h.hot // S, minlength=8), np.full(8, 2))
    base = wl.make_gate_inputs(8, 7168, wl.DSV3, hot_per_group=2, hot_shift=0.0)
    assert np.allclose(h.bias[h.hot] - base.bias[h.hot], wl.HOT_SHIFT, atol=1e-6)


def test_random_indices_distinct_rows():
    idx = wl.random_indices(100, 8, 32, seed=3)
    assert idx.shape == (100, 8) and idx.dtype == np.int32
    assert all(len(set(r)) == 8 for r in idx.tolist())
    assert idx.min() >= 0 and idx.max() < 32
