"""Plain CPU decode step of a pre-norm decoder stack with a per-session
cache: the definition the frame-synchronous batched step must reproduce.

Test infrastructure (see the package docstring).

What the step computes, with the pages it follows:

* Each session advances by exactly one frame per step; a frame is one
  decoder forward at the session's next position (PersonaPlex 7B page,
  "What Real-time Means for a Full-duplex Agent": the model processes one
  80 ms frame at a time).
* The sessions of a batch are independent; batching only shares the weight
  read (Nemotron VoiceChat case study, "The solution" and "Under the hood";
  the bandwidth blog, section 2 on concurrency).  So the batched step is S
  single-session steps; here the projections are done as one matrix product
  over the batch rows (a library primitive), which changes nothing per row.
* Weights and activations in bf16, temporal cache in FP8 (PersonaPlex
  page, "Compressing the Temporal KV cache"); the talker cache in fp32
  (Nemotron profile.json, serving_profile precision map).
* A session's window holds at most 1500 frames (profile.json,
  serving_profile context_steps).  Two readings of what happens after the
  window fills: the fixed window (default) refuses a further frame; the
  rolling window (``cfg["kv_ring"] = 1``) keeps the session going -- the
  vLLM-Omni recipe's realtime configuration ("Performance") leaves the
  session length unbounded -- and attends over the last ``max_context``
  frames only, each frame keeping its absolute index as its rotary
  position.
* The depth stack runs 8 sequential steps per frame (PersonaPlex page,
  "Predictable GPU execution").

The pages give no block diagram.  Readings used (the textbook pre-norm
decoder): RMSNorm x * (mean(x^2) + eps)^(-1/2) * g before attention and
before the FFN, residual adds after each, final RMSNorm on the output, no
biases; rotary embedding on adjacent pairs (2i, 2i+1) with angle
p * base^(-2i/D), the table computed in float64 and rounded to float32;
attention scale 1/sqrt(D), causal over 0..p including the new frame; query
head h reads kv head floor(h * H_kv / H_q); SwiGLU FFN silu(gate) * up.  With
an FP8 cache the new frame's key/value are stored as codes of k / sigma and
v / sigma (static per-(layer, K|V, kv-head) scales) and every position,
the new one included, is read back as sigma * decode(code).

Arithmetic is float32 by default (``dtype=np.float64`` for the rounding
check); inputs and weights are used exactly as given, and activations are
kept at that precision.  ``act_round="bf16"`` instead rounds every
projection input of the main stack (the normed rows before QKV and
gate/up, the attention output before O, the SwiGLU product before down) to
bf16, the activation type the PersonaPlex page names ("Compressing the
Temporal KV cache"): the method at its stated precision, whose distance from
the float64 step measures how far rounding at that precision moves a
session's output.
"""
from __future__ import annotations

import numpy as np

from . import fp8


# ----------------------------------------------------------------------------
# building blocks


def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float, dtype=np.float32) -> np.ndarray:
    """x * (mean(x^2) + eps)^(-1/2) * g over the last axis."""
    x = x.astype(dtype)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    r = (1.0 / np.sqrt(ms + dtype(eps))).astype(dtype)
    return (x * r * g.astype(dtype)).astype(dtype)


def rope_table(max_pos: int, head_dim: int, base: float, dtype=np.float32):
    """cos and sin of p * base^(-2i/D) for p < max_pos, i < D/2, evaluated
    in float64 and rounded once to ``dtype``: arrays [max_pos][D/2]."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    theta = base ** (-2.0 * i / head_dim)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * theta[None, :]
    return np.cos(ang).astype(dtype), np.sin(ang).astype(dtype)


def rope(x: np.ndarray, pos: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate the pairs (2i, 2i+1) of each head vector of x [n, H, D] by the
    angles of position pos[n]."""
    c = cos[pos][:, None, :]
    s = sin[pos][:, None, :]
    x0 = x[..., 0::2]
    x1 = x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Each value rounded once to the nearest bf16 number (8 significant
    bits, ties to the even one), in x's dtype: with x = m * 2^e and
    0.5 <= |m| < 1, m becomes a multiple of 2^-8.  (Values in bf16's normal
    range; zero, infinities and NaN pass through.)"""
    x = np.asarray(x)
    m, e = np.frexp(x.astype(np.float64))
    return np.ldexp(np.round(m * 256.0) / 256.0, e).astype(x.dtype)


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def quantize_rows(w: np.ndarray):
    """FP8 E4M3 weights with one scale per output row (an nn.Linear row):
    scale = max|row| / 448 in float32 (1 for a row of zeros), codes of
    w / scale, read back as scale * decode(code).  Returns (dequantized
    float32 weights, scales).  FP8 weights halve the bytes a decode step
    streams per parameter; the bandwidth blog measured the bf16 -> fp8 switch
    (section 2, and its section 6 question on quantization), where per-token
    fixed costs and the conversion back from 8 bits ate part of the gain."""
    w = np.asarray(w, dtype=np.float32)
    mx = np.max(np.abs(w), axis=1)
    sc = np.where(mx > 0, mx / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    codes = fp8.encode(w / sc[:, None])
    return (fp8.decode(codes, np.float32) * sc[:, None]).astype(np.float32), sc


# ----------------------------------------------------------------------------
# cache


class Cache:
    """Per-slot caches of one stack: ``kv[slot]`` is [L][2 (K|V)][H_kv][n][D],
    uint8 E4M3 codes for an FP8 cache, else values in the oracle dtype, with
    entry t holding the frame of absolute index t.  With a fixed window n is
    max_context; with a rolling window the history grows as frames arrive
    and reads cover the last max_context frames."""

    def __init__(self, n_layers: int, n_kv_heads: int, max_context: int, head_dim: int,
                 fp8_cache: bool, dtype=np.float32, rolling: bool = False):
        self.shape = (n_layers, 2, n_kv_heads, max_context, head_dim)
        self.window = max_context
        self.rolling = rolling
        self.fp8 = fp8_cache
        self.dtype = dtype
        self.kv: dict[int, np.ndarray] = {}

    def slot(self, s: int, upto: int = 0) -> np.ndarray:
        """The slot's history, grown (rolling window) to hold frames < upto."""
        if s not in self.kv:
            self.kv[s] = np.zeros(self.shape, dtype=np.uint8 if self.fp8 else self.dtype)
        c = self.kv[s]
        if upto > c.shape[3]:
            if not self.rolling:
                raise ValueError("frame index outside the fixed window")
            grown = np.zeros(c.shape[:3] + (max(upto, 2 * c.shape[3]),) + c.shape[4:], dtype=c.dtype)
            grown[:, :, :, :c.shape[3]] = c
            self.kv[s] = c = grown
        return c

    def store(self, s: int, layer: int, kv: int, pos: int, vec: np.ndarray, scale: np.ndarray):
        """Write the new frame's [H_kv][D] key or value at frame index ``pos``."""
        c = self.slot(s, pos + 1)
        if self.fp8:
            c[layer, kv, :, pos, :] = fp8.encode(vec.astype(np.float32) /
                                                 scale.astype(np.float32)[:, None])
        else:
            c[layer, kv, :, pos, :] = vec.astype(self.dtype)

    def prefill(self, s: int, layer: int, values: np.ndarray, scale: np.ndarray, t0: int = 0):
        """Fill frames t0..t0+n-1 of one layer from raw values [2][H_kv][n][D]
        stored the same way as new frames."""
        n = values.shape[2]
        c = self.slot(s, t0 + n)
        if self.fp8:
            c[layer, :, :, t0:t0 + n, :] = fp8.encode(values.astype(np.float32) /
                                                      scale.astype(np.float32)[:, :, None, None])
        else:
            c[layer, :, :, t0:t0 + n, :] = values.astype(self.dtype)

    def read(self, s: int, layer: int, kv: int, g: int, lo: int, hi: int, scale: float) -> np.ndarray:
        """Frames lo..hi-1 of kv-head g read back: [hi-lo][D] in the oracle dtype."""
        c = self.slot(s, hi)[layer, kv, g, lo:hi, :]
        if self.fp8:
            return fp8.decode(c, np.float32).astype(self.dtype) * self.dtype(scale)
        return c.astype(self.dtype)

    def first_attended(self, pos: int) -> int:
        """First frame index the frame at ``pos`` attends to: 0, or with a
        rolling window the start of the last ``window`` frames."""
        return max(0, pos + 1 - self.window) if self.rolling else 0


# ----------------------------------------------------------------------------
# one decoder stack, one frame


def _stack_step(x, pos, slots, layers, n_layers, shape, eps, cos, sin, cache, kv_scale,
                g_final, dtype, act=lambda v: v):
    """Advance rows x [n][d] (row i = slot slots[i] at new-frame index
    pos[i]) through ``n_layers`` layers; returns the final-normed output.
    ``act`` is applied to every projection input (rounding to the
    activation type, or nothing)."""
    hq, hkv, hd = shape
    n = x.shape[0]
    x = x.astype(dtype)
    inv_sqrt_d = dtype(1.0 / np.sqrt(hd))
    for l in range(n_layers):
        w = {k: v.astype(dtype) for k, v in layers(l).items()}
        a = act(rmsnorm(x, w["g_attn"], eps, dtype))
        q = (a @ w["wq"].T).reshape(n, hq, hd)
        k = (a @ w["wk"].T).reshape(n, hkv, hd)
        v = (a @ w["wv"].T).reshape(n, hkv, hd)
        q = rope(q, pos, cos, sin)
        k = rope(k, pos, cos, sin)
        o = np.empty((n, hq, hd), dtype=dtype)
        for i in range(n):
            s, p = int(slots[i]), int(pos[i])
            cache.store(s, l, 0, p, k[i], kv_scale[l, 0])
            cache.store(s, l, 1, p, v[i], kv_scale[l, 1])
            for h in range(hq):
                g = (h * hkv) // hq
                lo = cache.first_attended(p)
                kh = cache.read(s, l, 0, g, lo, p + 1, kv_scale[l, 0, g])
                vh = cache.read(s, l, 1, g, lo, p + 1, kv_scale[l, 1, g])
                sc = (kh @ q[i, h]) * inv_sqrt_d
                sc = sc - np.max(sc)
                e = np.exp(sc)
                wts = e / np.sum(e)
                o[i, h] = wts @ vh
        x = x + act(o.reshape(n, hq * hd)) @ w["wo"].T
        b = act(rmsnorm(x, w["g_ffn"], eps, dtype))
        hid = act(silu(b @ w["w_gate"].T) * (b @ w["w_up"].T))
        x = x + hid @ w["w_down"].T
    return rmsnorm(x, g_final, eps, dtype)


class Oracle:
    """Reference decode step for one configuration.

    ``model`` supplies float32 weights: ``layer(l)`` -> dict with wq, wk, wv,
    wo, w_gate, w_up, w_down ([out, in]) and g_attn, g_ffn; attributes
    g_final, kv_scale [L][2][H_kv] (ignored for fp32 caches), and for a
    depth stack w_in, depth_layer(l), depth_g_final.
    """

    def __init__(self, cfg: dict, model, dtype=np.float32, act_round: str | None = None):
        if act_round not in (None, "bf16"):
            raise ValueError("act_round is None or 'bf16'")
        self.cfg = cfg
        self.model = model
        self.dtype = dtype
        self.act = round_bf16 if act_round == "bf16" else (lambda v: v)
        self.rolling = bool(cfg.get("kv_ring", 0))
        self.cache = Cache(cfg["n_layers"], cfg["n_kv_heads"], cfg["max_context"],
                           cfg["head_dim"], cfg["kv_dtype"] == "fp8", dtype, rolling=self.rolling)
        self.cos, self.sin = rope_table(cfg["max_context"], cfg["head_dim"], cfg["rope_base"], dtype)
        if cfg["kv_dtype"] == "fp8":
            self.kv_scale = np.asarray(model.kv_scale, dtype=np.float32)
        else:
            self.kv_scale = np.ones((cfg["n_layers"], 2, cfg["n_kv_heads"]), dtype=np.float32)
        self.depth = cfg.get("depth_steps", 0) > 0
        # FP8 weights: every projection (and the head) used as scale * decode(code)
        self.w8 = cfg["w_dtype"] == "fp8"
        self._qlayers: dict = {}
        if self.depth:
            if cfg["kv_dtype"] != "f32":
                raise ValueError("the depth stack is defined with an fp32 cache only")
            self.dcos, self.dsin = rope_table(cfg["depth_steps"], cfg["depth_head_dim"],
                                              cfg["rope_base"], dtype)

    def step(self, slots, x, pos):
        """One frame for the active rows: slots[i] at new-frame index pos[i]
        with input x[i].  Writes the new cache entries; returns y [n][d] and,
        with a depth stack, the depth outputs [n][steps][depth_d]."""
        cfg = self.cfg
        slots = np.asarray(slots, dtype=np.int64)
        pos = np.asarray(pos, dtype=np.int64)
        if np.any(pos < 0) or (not self.rolling and np.any(pos >= cfg["max_context"])):
            raise ValueError("position outside the context window")
        if pos.size and int(pos.max()) >= self.cos.shape[0]:  # rolling window: rotary angles further out
            self.cos, self.sin = rope_table(2 * int(pos.max()) + 2, cfg["head_dim"], cfg["rope_base"],
                                            self.dtype)
        y = _stack_step(np.asarray(x), pos, slots, self.layer, cfg["n_layers"],
                        (cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"]), cfg["rms_eps"],
                        self.cos, self.sin, self.cache, self.kv_scale, self.model.g_final,
                        self.dtype, self.act)
        if not self.depth:
            return y
        return y, self.depth_loop(y)

    def depth_loop(self, y):
        """Per-frame inner loop: c = W_in y; z_{-1} = 0; for k in 0..steps-1
        run the depth stack on c + z_{k-1} at depth position k over a cache
        holding only this frame's depth positions; emit z_k."""
        cfg = self.cfg
        n = y.shape[0]
        dt = self.dtype
        c = y.astype(dt) @ self.model.w_in.astype(dt).T
        dcache = Cache(cfg["depth_layers"], cfg["depth_kv_heads"], cfg["depth_steps"],
                       cfg["depth_head_dim"], False, dt)
        ones = np.ones((cfg["depth_layers"], 2, cfg["depth_kv_heads"]), dtype=np.float32)
        z = np.zeros((n, cfg["depth_d"]), dtype=dt)
        out = np.empty((n, cfg["depth_steps"], cfg["depth_d"]), dtype=dt)
        rows = np.arange(n)
        for k in range(cfg["depth_steps"]):
            z = _stack_step(c + z, np.full(n, k, dtype=np.int64), rows, self.model.depth_layer,
                            cfg["depth_layers"],
                            (cfg["depth_heads"], cfg["depth_kv_heads"], cfg["depth_head_dim"]),
                            cfg["rms_eps"], self.dcos, self.dsin, dcache, ones,
                            self.model.depth_g_final, dt)
            out[:, k] = z
        return out

    def layer(self, l: int) -> dict:
        """Weights of main-stack layer l as the step uses them."""
        w = self.model.layer(l)
        if not self.w8:
            return w
        if l not in self._qlayers:
            q = dict(w)
            for n in ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down"):
                q[n] = quantize_rows(w[n])[0]
            self._qlayers[l] = q
        return self._qlayers[l]

    def head(self, y):
        """Output head after the step: logits = y . W_head^T over the
        vocabulary and the greedy token (the vLLM-Omni recipe: one text token
        per acoustic frame, "Summary"; sampling greedy end to end, "Key
        flags").  Ties go to the lowest token index.  Returns (logits [n][V],
        tokens [n])."""
        dt = self.dtype
        wh = quantize_rows(self.model.w_head)[0] if self.w8 else self.model.w_head
        logits = np.asarray(y).astype(dt) @ wh.astype(dt).T
        return logits, np.argmax(logits, axis=1)

    def prefill(self, slot: int, layer: int, values: np.ndarray, t0: int = 0):
        """Fill frames t0..t0+n-1 of ``slot`` at ``layer`` from raw key/value
        vectors [2][H_kv][n][D] (quantised like new frames)."""
        self.cache.prefill(slot, layer, values, self.kv_scale[layer], t0)
