"""Upload of the synthetic weights to the GPU as torch tensors in the
layout the library's C ABI takes (nn.Linear [out, in], bf16 or fp32
matrices; fp32 gains and FP8 scales).  Plumbing only: values are copied,
bf16 weights are already bf16-representable so the cast is exact."""
from __future__ import annotations

import numpy as np
import torch

from . import LAYER_MATS


def _mat(a: np.ndarray, wdt, device):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device=device, dtype=wdt)


def _f32(a: np.ndarray, device):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def _layer(w: dict, wdt, device) -> dict:
    out = {n: _mat(w[n], wdt, device) for n in LAYER_MATS}
    out["g_attn"] = _f32(w["g_attn"], device)
    out["g_ffn"] = _f32(w["g_ffn"], device)
    return out


def device_weights(model, device="cuda") -> dict:
    """All weights of ``model`` (a synth.Model) as device tensors."""
    cfg = model.cfg
    wdt = torch.bfloat16 if cfg["w_dtype"] in ("bf16", "fp8") else torch.float32
    out = {
        "layers": [_layer(model.layer(l), wdt, device) for l in range(cfg["n_layers"])],
        "g_final": _f32(model.g_final, device),
        "kv_scale": _f32(model.kv_scale, device) if cfg["kv_dtype"] == "fp8" else None,
    }
    if cfg.get("depth_steps", 0):
        out["w_in"] = _mat(model.w_in, wdt, device)
        out["depth_layers"] = [_layer(model.depth_layer(l), wdt, device)
                               for l in range(cfg["depth_layers"])]
        out["depth_g_final"] = _f32(model.depth_g_final, device)
    if cfg.get("vocab", 0):
        out["w_head"] = _mat(model.w_head, wdt, device)
    return out


def random_device_weights(cfg: dict, seed: int = 0, device="cuda") -> dict:
    """Weights of the same distributions (matrices ~N(0, 0.02) in the
    config's weight type, gains 1, FP8 scales as in ``synth.kv_scales``)
    drawn directly on the GPU from torch's seeded generator.  Used where the
    values need not equal the host generator's (timing runs)."""
    from . import kv_scales, weight_shape
    wdt = torch.bfloat16 if cfg["w_dtype"] in ("bf16", "fp8") else torch.float32
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)

    def mat(name, depth=False):
        shape = weight_shape(cfg, name, depth=depth)
        t = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
        return t.mul_(0.02).to(wdt)

    def layer(depth=False):
        d = cfg["depth_d"] if depth else cfg["d_model"]
        out = {n: mat(n, depth) for n in LAYER_MATS}
        out["g_attn"] = torch.ones(d, device=device)
        out["g_ffn"] = torch.ones(d, device=device)
        return out

    out = {
        "layers": [layer() for _ in range(cfg["n_layers"])],
        "g_final": torch.ones(cfg["d_model"], device=device),
        "kv_scale": _f32(kv_scales(cfg), device) if cfg["kv_dtype"] == "fp8" else None,
    }
    if cfg.get("depth_steps", 0):
        out["w_in"] = mat("w_in")
        out["depth_layers"] = [layer(True) for _ in range(cfg["depth_layers"])]
        out["depth_g_final"] = torch.ones(cfg["depth_d"], device=device)
    if cfg.get("vocab", 0):
        out["w_head"] = mat("w_head")
    return out
