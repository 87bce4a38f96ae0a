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
    wdt = torch.bfloat16 if cfg["w_dtype"] == "bf16" else torch.float32
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
    return out
