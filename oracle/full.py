"""Full causal recompute of one session: the whole frame sequence through
the stack at once, with a causal mask instead of a cache.

Test infrastructure (see the package docstring).

Processing a stream frame by frame with cached keys/values must give, at
every frame, the same result as recomputing the causal forward over all
frames so far: each frame is computed once and never revisited (the
bandwidth blog, section 4 on cache-aware streaming recognition, and the
interview answer on it in section 6).  This module is that recompute,
written as matrix products over the whole sequence [T][d] with a causal
mask, so it shares no attention or cache-indexing code with the step (with
a rolling window the mask also drops frames max_context or more back).  The
cache's storage rounding (FP8 codes of x / sigma read back as sigma * decode)
is applied to the full key/value matrices, since the cache is what the
attention reads.
"""
from __future__ import annotations

import numpy as np

from . import fp8
from .decoder import rmsnorm, rope_table, silu


def _rope_rows(x, cos, sin):
    """x [T][H][D]; row t rotated by the angles of position t."""
    t = x.shape[0]
    c = cos[:t][:, None, :]
    s = sin[:t][:, None, :]
    out = np.empty_like(x)
    out[..., 0::2] = x[..., 0::2] * c - x[..., 1::2] * s
    out[..., 1::2] = x[..., 0::2] * s + x[..., 1::2] * c
    return out


def _stack_full(X, layers, n_layers, shape, eps, base, g_final, kv_scale, fp8_cache, dtype,
                window=None):
    hq, hkv, hd = shape
    T = X.shape[0]
    cos, sin = rope_table(T, hd, base, dtype)
    X = X.astype(dtype)
    i = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    mask = j > i  # True = not attended: the future
    if window is not None:  # and, with a rolling window, frames window or more back
        mask = mask | (j <= i - window)
    for l in range(n_layers):
        w = {k: v.astype(dtype) for k, v in layers(l).items()}
        A = rmsnorm(X, w["g_attn"], eps, dtype)
        Q = _rope_rows((A @ w["wq"].T).reshape(T, hq, hd), cos, sin)
        K = _rope_rows((A @ w["wk"].T).reshape(T, hkv, hd), cos, sin)
        V = (A @ w["wv"].T).reshape(T, hkv, hd)
        if fp8_cache:
            sk = kv_scale[l, 0].astype(np.float32)[None, :, None]
            sv = kv_scale[l, 1].astype(np.float32)[None, :, None]
            K = fp8.decode(fp8.encode(K.astype(np.float32) / sk)).astype(dtype) * sk.astype(dtype)
            V = fp8.decode(fp8.encode(V.astype(np.float32) / sv)).astype(dtype) * sv.astype(dtype)
        O = np.empty((T, hq, hd), dtype=dtype)
        for h in range(hq):
            g = (h * hkv) // hq
            S = (Q[:, h, :] @ K[:, g, :].T) / dtype(np.sqrt(hd))
            S = np.where(mask, -np.inf, S)
            S = S - S.max(axis=1, keepdims=True)
            P = np.exp(S)
            P = P / P.sum(axis=1, keepdims=True)
            O[:, h, :] = P @ V[:, g, :]
        X = X + O.reshape(T, hq * hd) @ w["wo"].T
        B = rmsnorm(X, w["g_ffn"], eps, dtype)
        X = X + (silu(B @ w["w_gate"].T) * (B @ w["w_up"].T)) @ w["w_down"].T
    return rmsnorm(X, g_final, eps, dtype)


def forward_full(cfg: dict, model, X: np.ndarray, dtype=np.float32) -> np.ndarray:
    """Outputs [T][d] of the main stack for one session's frames X [T][d]
    starting at position 0 (with ``cfg["kv_ring"]``, each frame attends to
    the last ``max_context`` frames only)."""
    fp8_cache = cfg["kv_dtype"] == "fp8"
    scale = np.asarray(model.kv_scale, dtype=np.float32) if fp8_cache else None
    window = cfg["max_context"] if cfg.get("kv_ring", 0) else None
    return _stack_full(X, model.layer, cfg["n_layers"],
                       (cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"]), cfg["rms_eps"],
                       cfg["rope_base"], model.g_final, scale, fp8_cache, dtype, window)


def depth_full(cfg: dict, model, Xd: np.ndarray, dtype=np.float32) -> np.ndarray:
    """Depth-stack outputs [K][depth_d] for one frame's depth inputs Xd
    [K][depth_d] (teacher-forced: row k is c + z_{k-1})."""
    return _stack_full(Xd, model.depth_layer, cfg["depth_layers"],
                       (cfg["depth_heads"], cfg["depth_kv_heads"], cfg["depth_head_dim"]),
                       cfg["rms_eps"], cfg["rope_base"], model.depth_g_final, None, False, dtype)
