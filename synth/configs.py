"""Workload shapes of the frame-synchronous decode step.

Each entry names one stack and batch: decoder shape, slot capacity, context
window, storage types and the new-frame position(s) the workload steps at.
Depth-stack fields describe the per-frame inner loop of the talker-shaped
workload (8 sequential steps of a 6-layer stack, cache cleared each frame).
"""
from __future__ import annotations

import copy

_BASE = dict(
    rms_eps=1e-6,
    rope_base=10000.0,
    max_context=1500,
    depth_steps=0, depth_layers=0, depth_d=0, depth_heads=0, depth_kv_heads=0,
    depth_head_dim=0, depth_ffn=0,
    kv_ring=0,
    vocab=0,
)

_7B = dict(n_layers=32, d_model=4096, n_heads=32, n_kv_heads=32, head_dim=128, d_ffn=11264,
           w_dtype="bf16", act_dtype="bf16", kv_dtype="fp8")

CONFIGS = {
    # 2 layers, d 256, 4x64 MHA, FFN 1024, fp32 throughout; 2 sessions x 16
    # frames decoded from an empty cache.
    "tiny": dict(_BASE, n_layers=2, d_model=256, n_heads=4, n_kv_heads=4, head_dim=64,
                 d_ffn=1024, w_dtype="f32", act_dtype="f32", kv_dtype="f32",
                 max_slots=2, n_frames=16),
    # 7B-class temporal stack, 8 sessions, new frame at index 256.
    "7b_s8_p256": dict(_BASE, **_7B, max_slots=8, position=256),
    # 7B-class stack, 80 sessions, new frame at index 1499 (full 120 s window).
    "7b_s80_p1499": dict(_BASE, **_7B, max_slots=80, position=1499),
    # 7B-class stack, 80 slots, 56 active with lengths U{1..1500}.
    "7b_ragged_80x56": dict(_BASE, **_7B, max_slots=80, n_active=56),
    # Talker-shaped fp32 stack, GQA 4:1 with head_dim 256, 56 sessions at
    # 1500 frames, plus the 8-step depth loop of a 6-layer d=1024 stack.
    "talker_s56": dict(_BASE, n_layers=26, d_model=1152, n_heads=4, n_kv_heads=1, head_dim=256,
                       d_ffn=6912, w_dtype="f32", act_dtype="f32", kv_dtype="f32",
                       max_slots=56, position=1499,
                       depth_steps=8, depth_layers=6, depth_d=1024, depth_heads=8,
                       depth_kv_heads=8, depth_head_dim=128, depth_ffn=2816),
}


def get_config(name: str) -> dict:
    return copy.deepcopy(CONFIGS[name])


def scaled_config(name: str, **over) -> dict:
    """A copy of a named workload with some fields replaced (smaller layer
    count, fewer slots, shorter window...) for tests that must finish fast
    while keeping the same head and dtype structure."""
    cfg = get_config(name)
    cfg.update(over)
    return cfg
