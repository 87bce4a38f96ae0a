"""The bench's roofline arithmetic reproduces the pages' own worked numbers
(tests/golden/bandwidth_blog_points.json, each with its page and section),
and the byte counts of the workloads match their closed forms."""
import json
import os

import pytest

import synth
from frame_decode_amd import roofline as rf

G = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "bandwidth_blog_points.json")))


def test_decode_rate_ceiling():
    g = G["upper_bound_tok_s"]
    assert abs(rf.tokens_per_s_upper_bound(g["bandwidth_gbs"], g["weight_gb"]) - g["printed"]) < g["tolerance"] + 0.35


def test_bandwidth_share():
    g = G["bandwidth_share"]
    used = g["rate_tok_s"] * g["weight_gb"]
    assert round(used) == g["printed_gbs"]
    assert round(100 * rf.bandwidth_share(g["rate_tok_s"], g["weight_gb"], g["bandwidth_gbs"])) == g["printed_pct"]


@pytest.mark.parametrize("key", ["crossover_bf16", "crossover_fp8"])
def test_compute_crossover(key):
    g = G[key]
    b = rf.compute_crossover_batch(g["tflops"], g["bandwidth_gbs"], g["bytes_per_param"])
    assert abs(b - g["printed"]) <= g["tolerance"]


def test_batched_compute_share():
    g = G["batched_compute_4b"]
    tf = 2 * g["params_b"] * 1e9 * g["tok_s"] / 1e12
    assert round(tf, 1) == g["printed_tflops"]
    assert round(100 * tf / g["measured_tflops"]) == g["printed_pct_of_measured"]


def test_case_study_numbers():
    assert round(100 * (1 - 1 / G["cost_reduction_56"]["sessions"]), 1) == G["cost_reduction_56"]["printed_pct"]
    w = G["window"]
    assert w["steps"] * w["step_ms"] / 1000 == w["printed_seconds"]
    p = G["p99_reduction"]
    for ours, ref, pct in zip(p["ours_ms"], p["ref_ms"], p["printed_pct"]):
        assert round(100 * (1 - ours / ref), 1) == pct


def test_workload_bytes():
    c3 = synth.get_config("7b_s80_p1499")
    assert rf.weight_bytes(c3) == 13_153_337_344
    assert rf.kv_bytes_per_position(c3) == 262_144
    assert rf.step_bytes(c3, [1499] * 80) == 44_610_617_344
    assert rf.attention_bytes_per_launch(c3, [1499] * 80) == 983_040_000
    c2 = synth.get_config("7b_s8_p256")
    assert rf.step_bytes(c2, [256] * 8) == 13_692_305_408
    c5 = synth.get_config("talker_s56")
    # main 2,791,047,168 + depth 8 x 308,281,344 + W_in 4,718,592 weights, fp32 cache 56 x 1500 x 26 x 2 x 256 x 4
    assert rf.weight_bytes(c5) == 2_791_047_168 + 8 * 308_281_344 + 4_718_592
    assert rf.step_bytes(c5, [1499] * 56) == 9_734_848_512
    # at 8 TB/s the 80-session, 1500-frame step takes 5.576 ms
    assert abs(rf.roofline_seconds(44_610_617_344) * 1e3 - 5.576) < 1e-3


def test_rolling_window_bytes_cap_at_the_window():
    """With a rolling window a session past the window streams exactly one
    window of cache per layer, the same bytes as a session at the window's
    last frame."""
    import synth
    from frame_decode_amd import roofline as rf
    cfg = synth.get_config("7b_s80_p1499")
    ring = dict(cfg, kv_ring=1)
    assert rf.attended(ring, 5000) == 1500 and rf.attended(ring, 20) == 21
    assert rf.attended(cfg, 20) == 21
    assert rf.step_bytes(ring, [4999] * 80) == rf.step_bytes(cfg, [1499] * 80) == 44_610_617_344
    assert rf.attention_bytes_per_launch(ring, [3000] * 80) == 983_040_000
