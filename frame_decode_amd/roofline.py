"""Roofline arithmetic of the decode step (host-side report logic).

The decode step is bound by memory bandwidth: every weight byte is read
once per step no matter how many sessions share it, so frames/s <= bandwidth
/ bytes per step (the bandwidth blog, section 2, "Principle"; its interview
answer on estimating the generation limit).  Batching sessions shares the
weight read, and compute only binds once 2 FLOP per parameter per session
outgrow the bandwidth (same page, section 2 on concurrent requests).  Here
the bytes per step are one read of every weight plus a read of every cached
position of every active session (the cache is what attention streams) and
the write of the new entries.
"""
from __future__ import annotations

MI355X_HBM_PEAK_GBS = 8000.0  # GB/s, published HBM3E peak
MI355X_BF16_DENSE_TFLOPS = 2500.0
MI355X_FP32_TFLOPS = 157.3


def weight_params(cfg: dict, depth: bool = False) -> int:
    if depth:
        d, hq, hkv, hd, f, L = (cfg["depth_d"], cfg["depth_heads"], cfg["depth_kv_heads"],
                                cfg["depth_head_dim"], cfg["depth_ffn"], cfg["depth_layers"])
    else:
        d, hq, hkv, hd, f, L = (cfg["d_model"], cfg["n_heads"], cfg["n_kv_heads"],
                                cfg["head_dim"], cfg["d_ffn"], cfg["n_layers"])
    per_layer = (hq + 2 * hkv) * hd * d + d * hq * hd + 3 * d * f
    return L * per_layer


def weight_bytes(cfg: dict, head: bool = False) -> int:
    """One read of every projection weight of the main stack (and, with a
    depth stack, its weights once per depth step plus the input projection;
    with head=True the output head's vocab x d_model weights)."""
    wb = {"bf16": 2, "fp8": 1}.get(cfg["w_dtype"], 4)
    b = weight_params(cfg) * wb
    if cfg["w_dtype"] == "fp8":  # one fp32 scale per output row of every projection
        d, hq, hkv, hd, f = cfg["d_model"], cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"], cfg["d_ffn"]
        b += 4 * cfg["n_layers"] * ((hq + 2 * hkv) * hd + d + 2 * f + d)
    if cfg.get("depth_steps", 0):
        b += cfg["depth_steps"] * weight_params(cfg, depth=True) * wb
        b += cfg["depth_d"] * cfg["d_model"] * wb
    if head:
        b += cfg.get("vocab", 0) * cfg["d_model"] * wb
    return b


def kv_bytes_per_position(cfg: dict) -> int:
    """Cache bytes of one position of one session over all layers (K and V)."""
    eb = 1 if cfg["kv_dtype"] == "fp8" else 4
    return cfg["n_layers"] * 2 * cfg["n_kv_heads"] * cfg["head_dim"] * eb


def attended(cfg: dict, p: int) -> int:
    """Cached positions the frame at index p attends over: p + 1, capped at
    the window with a rolling window (kv_ring)."""
    n = int(p) + 1
    return min(n, cfg["max_context"]) if cfg.get("kv_ring", 0) else n


def step_bytes(cfg: dict, positions, head: bool = False) -> int:
    """Algorithmic bytes of one step: weights once, plus for each active
    session the cached positions it attends over (the new entry is written
    and read once; counted once); head=True adds the output head's weights."""
    kvp = kv_bytes_per_position(cfg)
    return weight_bytes(cfg, head) + sum(attended(cfg, p) * kvp for p in positions)


def attention_bytes_per_launch(cfg: dict, positions) -> int:
    """Bytes one attention launch (one layer) streams: K and V of every
    cached position of every active session."""
    eb = 1 if cfg["kv_dtype"] == "fp8" else 4
    return sum(attended(cfg, p) for p in positions) * 2 * cfg["n_kv_heads"] * cfg["head_dim"] * eb


def step_flops(cfg: dict, n_sessions: int) -> float:
    """2 FLOP per weight parameter per session row (plus attention)."""
    return 2.0 * weight_params(cfg) * n_sessions


def roofline_seconds(nbytes: float, peak_gbs: float = MI355X_HBM_PEAK_GBS) -> float:
    return nbytes / (peak_gbs * 1e9)


def tokens_per_s_upper_bound(bandwidth_gbs: float, weight_gb: float) -> float:
    """Decode-rate ceiling when every weight byte is read once per token."""
    return bandwidth_gbs / weight_gb


def bandwidth_share(rate: float, weight_gb: float, bandwidth_gbs: float) -> float:
    """Fraction of the bandwidth a decode rate uses (rate x bytes / bandwidth)."""
    return rate * weight_gb / bandwidth_gbs


def compute_crossover_batch(flops_tflops: float, bandwidth_gbs: float, bytes_per_param: float) -> float:
    """Concurrent sequences beyond which 2 FLOP/param/sequence exceed what
    the bandwidth-bound weight read allows: (F / B) * bytes_per_param / 2."""
    return flops_tflops * 1e12 / (bandwidth_gbs * 1e9) * bytes_per_param / 2.0


def max_sessions_by_time(step_budget_s: float, achieved_gbs: float, weight_b: float,
                         kv_per_session_b: float) -> float:
    return (step_budget_s * achieved_gbs * 1e9 - weight_b) / kv_per_session_b


def max_sessions_by_capacity(hbm_bytes: float, weight_b: float, other_b: float,
                             kv_per_session_b: float) -> float:
    return (hbm_bytes - weight_b - other_b) / kv_per_session_b
