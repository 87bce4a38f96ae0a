"""Seeded synthetic inputs for the frame-synchronous decode step.

This module is the only code shared by the HIP path's tests/bench and by the
oracle's tests.  It holds the workload shapes and the seeded random draws
(weights, frame embeddings, cache prefill values, FP8 scales, ragged slot
sets) and nothing of the decode method itself: no normalisation, no rotary
embedding, no attention, no FP8 encoding.

Distributions follow the stated workloads: weight matrices ~N(0, 0.02),
frame embeddings ~N(0, 1), cache prefill ~N(0, (0.02*sqrt(d_model))^2) (the
spread of a projection of a unit-RMS vector through such weights), norm gains
1 (or 1 + N(0, 0.02) when gain noise is requested), FP8 scales
u * 6 * (0.02*sqrt(d_model)) / 448 with u ~ U[1, 2].

Seeds: 0 weights and gains, 1 frame embeddings keyed by (session, frame),
2 cache prefill keyed by (session, layer), 3 ragged active set and lengths,
4 FP8 scales.  Every draw is keyed by what it describes (session id, layer,
matrix name, row chunk), never by thread or slot, so any subset can be
regenerated on its own and the values do not depend on how many threads made
them.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .configs import CONFIGS, get_config, scaled_config  # noqa: F401

SEED_WEIGHTS = 0
SEED_INPUTS = 1
SEED_PREFILL = 2
SEED_RAGGED = 3
SEED_SCALES = 4

# Stable ids for the per-layer tensors, used as SeedSequence keys.
_NAME_ID = {
    "wq": 1, "wk": 2, "wv": 3, "wo": 4, "w_gate": 5, "w_up": 6, "w_down": 7,
    "g_attn": 8, "g_ffn": 9, "g_final": 10, "w_in": 11, "w_head": 12,
}
_DEPTH_OFFSET = 1000  # layer key offset for the depth stack's layers
_FINAL_LAYER_KEY = 999_999

_ROWS_PER_CHUNK_ELEMS = 1 << 22  # elements per independently seeded chunk


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def round_to_bf16(a: np.ndarray, out: np.ndarray | None = None) -> np.ndarray:
    """Round finite float32 values to the nearest bfloat16 (ties to even),
    returned as float32.  This is the storage format of the bf16 workloads'
    weights and inputs, applied once when the inputs are made."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    r = (u >> 16) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u  # finite inputs: no 32-bit overflow
    r &= np.uint32(0xFFFF0000)
    if out is not None:
        out.view(np.uint32)[...] = r
        return out
    return r.view(np.float32)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bf16-representable."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    return (a.view(np.uint32) >> 16).astype(np.uint16)


def _normal_chunked(key: list[int], shape: tuple[int, ...], std: float,
                    pool: ThreadPoolExecutor | None, bf16: bool = False) -> np.ndarray:
    rows = shape[0]
    cols = int(np.prod(shape[1:])) if len(shape) > 1 else 1
    out = np.empty((rows, cols), dtype=np.float32)
    rpc = max(1, _ROWS_PER_CHUNK_ELEMS // max(cols, 1))
    starts = list(range(0, rows, rpc))

    def fill(ci_r0):
        ci, r0 = ci_r0
        r1 = min(rows, r0 + rpc)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(key + [ci])))
        blk = out[r0:r1]
        g.standard_normal(out=blk, dtype=np.float32)
        blk *= np.float32(std)
        if bf16:
            round_to_bf16(blk, out=blk)

    items = list(enumerate(starts))
    if pool is None or len(items) == 1:
        for it in items:
            fill(it)
    else:
        list(pool.map(fill, items))
    return out.reshape(shape)


def matrix(cfg: dict, layer: int, name: str, *, depth: bool = False,
           pool: ThreadPoolExecutor | None = None) -> np.ndarray:
    """One weight matrix in nn.Linear [out, in] layout, float32 values
    (bf16-representable when the config's weights are bf16)."""
    shape = weight_shape(cfg, name, depth=depth)
    lk = layer + (_DEPTH_OFFSET if depth else 0)
    return _normal_chunked([SEED_WEIGHTS, lk, _NAME_ID[name]], shape, 0.02, pool,
                           bf16=cfg["w_dtype"] in ("bf16", "fp8"))  # (FP8: bf16 sources)


def gain(cfg: dict, layer: int, name: str, *, depth: bool = False,
         noise: bool = False) -> np.ndarray:
    d = cfg["depth_d"] if depth else cfg["d_model"]
    if not noise:
        g = np.ones(d, dtype=np.float32)
    else:
        lk = layer + (_DEPTH_OFFSET if depth else 0)
        r = np.random.Generator(np.random.PCG64(
            np.random.SeedSequence([SEED_WEIGHTS, lk, _NAME_ID[name], 7])))
        g = (1.0 + 0.02 * r.standard_normal(d)).astype(np.float32)
    if cfg["w_dtype"] in ("bf16", "fp8"):
        g = round_to_bf16(g)
    return g


def weight_shape(cfg: dict, name: str, *, depth: bool = False) -> tuple[int, int]:
    if depth:
        d, hq, hkv, hd, f = (cfg["depth_d"], cfg["depth_heads"], cfg["depth_kv_heads"],
                             cfg["depth_head_dim"], cfg["depth_ffn"])
    else:
        d, hq, hkv, hd, f = (cfg["d_model"], cfg["n_heads"], cfg["n_kv_heads"],
                             cfg["head_dim"], cfg["d_ffn"])
    return {
        "wq": (hq * hd, d), "wk": (hkv * hd, d), "wv": (hkv * hd, d),
        "wo": (d, hq * hd), "w_gate": (f, d), "w_up": (f, d), "w_down": (d, f),
        "w_in": (cfg.get("depth_d", 0), cfg["d_model"]),
        "w_head": (cfg.get("vocab", 0), cfg["d_model"]),
    }[name]


LAYER_MATS = ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")


def layer_weights(cfg: dict, layer: int, *, depth: bool = False, gain_noise: bool = False,
                  pool: ThreadPoolExecutor | None = None) -> dict:
    out = {n: matrix(cfg, layer, n, depth=depth, pool=pool) for n in LAYER_MATS}
    out["g_attn"] = gain(cfg, layer, "g_attn", depth=depth, noise=gain_noise)
    out["g_ffn"] = gain(cfg, layer, "g_ffn", depth=depth, noise=gain_noise)
    return out


def kv_scales(cfg: dict) -> np.ndarray:
    """Per-(layer, K|V, kv-head) FP8 scales, float32 [L][2][H_kv].  For
    float32 caches the scales are all 1 (unused)."""
    L, hkv = cfg["n_layers"], cfg["n_kv_heads"]
    if cfg["kv_dtype"] != "fp8":
        return np.ones((L, 2, hkv), dtype=np.float32)
    r = np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED_SCALES])))
    u = r.uniform(1.0, 2.0, size=(L, 2, hkv))
    return (u * 6.0 * (0.02 * np.sqrt(cfg["d_model"])) / 448.0).astype(np.float32)


class Model:
    """Lazily generated weights of one configuration.

    ``layer(l)`` returns the float32 weights of layer ``l`` (generated on
    first use and cached unless ``cache=False``); ``depth_layer(l)`` the same
    for the depth stack.  ``g_final``, ``depth_g_final``, ``w_in``, ``w_head``
    (output head, with a vocabulary) and ``kv_scale`` are attributes.
    """

    def __init__(self, cfg: dict, *, gain_noise: bool = False, cache: bool = True,
                 threads: int | None = None, zero: tuple[str, ...] = ()):
        self.cfg = cfg
        self.gain_noise = gain_noise
        self.cache = cache
        self._zero = set(zero)
        self._pool = ThreadPoolExecutor(max_workers=threads or _threads())
        self._layers: dict = {}
        self._depth: dict = {}
        self.g_final = gain(cfg, _FINAL_LAYER_KEY, "g_final", noise=gain_noise)
        self.kv_scale = kv_scales(cfg)
        if cfg.get("depth_steps", 0):
            self.w_in = matrix(cfg, 0, "w_in", pool=self._pool)
            self.depth_g_final = gain(cfg, _FINAL_LAYER_KEY, "g_final", depth=True,
                                      noise=gain_noise)
        else:
            self.w_in = None
            self.depth_g_final = None
        self.w_head = matrix(cfg, 0, "w_head", pool=self._pool) if cfg.get("vocab", 0) else None

    def _apply_zero(self, w: dict) -> dict:
        for n in self._zero:
            w[n] = np.zeros_like(w[n])
        return w

    def layer(self, l: int) -> dict:
        if l in self._layers:
            return self._layers[l]
        w = self._apply_zero(layer_weights(self.cfg, l, gain_noise=self.gain_noise,
                                           pool=self._pool))
        if self.cache:
            self._layers[l] = w
        return w

    def depth_layer(self, l: int) -> dict:
        if l in self._depth:
            return self._depth[l]
        w = self._apply_zero(layer_weights(self.cfg, l, depth=True, gain_noise=self.gain_noise,
                                           pool=self._pool))
        if self.cache:
            self._depth[l] = w
        return w

    def close(self):
        self._pool.shutdown(wait=False)


def frame_input(cfg: dict, session: int, frame: int) -> np.ndarray:
    """Input frame embedding e ~ N(0, 1) for (session id, frame index)."""
    r = np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED_INPUTS, session, frame])))
    e = r.standard_normal(cfg["d_model"], dtype=np.float32)
    if cfg["act_dtype"] == "bf16":
        e = round_to_bf16(e)
    return e


def frame_inputs(cfg: dict, sessions, frame_of) -> np.ndarray:
    """Stack of frame inputs: row i is session ``sessions[i]`` at frame
    ``frame_of[i]``."""
    return np.stack([frame_input(cfg, s, f) for s, f in zip(sessions, frame_of)])


def kv_std(cfg: dict) -> float:
    return 0.02 * float(np.sqrt(cfg["d_model"]))


def prefill_values(cfg: dict, session: int, layer: int, n_pos: int) -> np.ndarray:
    """Raw (unquantised) key/value vectors that fill positions 0..n_pos-1 of
    one session's cache at one layer: float32 [2 (K|V)][H_kv][n_pos][D].
    Each side stores them in its own cache format."""
    shape = (2, cfg["n_kv_heads"], n_pos, cfg["head_dim"])
    if n_pos == 0:
        return np.zeros(shape, dtype=np.float32)
    return _normal_chunked([SEED_PREFILL, session, layer], (shape[0] * shape[1] * n_pos, shape[3]),
                           kv_std(cfg), None).reshape(shape)


def ragged_slots(cfg: dict, n_active: int) -> tuple[np.ndarray, np.ndarray]:
    """Seeded active subset (sorted slot ids) and context lengths L_i ~
    U{1..max_context} for a ragged batch."""
    r = np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED_RAGGED])))
    slots = np.sort(r.choice(cfg["max_slots"], size=n_active, replace=False)).astype(np.int32)
    lengths = r.integers(1, cfg["max_context"] + 1, size=n_active).astype(np.int32)
    return slots, lengths
