"""Shared helpers of the GPU parity tests: build a device context from a
synthetic model, run the library and the oracle on the same seeded inputs,
and compare them."""
from __future__ import annotations

import sys

import numpy as np
import torch

import synth
from synth.device import device_weights


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def act_torch(cfg):
    return torch.bfloat16 if cfg["act_dtype"] == "bf16" else torch.float32


def make_context(cfg, model):
    from frame_decode_amd import Context
    w = device_weights(model)
    ctx = Context(cfg, w)
    torch.cuda.synchronize()
    del w
    return ctx


def rows_input(cfg, slot_session, slot_frame):
    """x_in [S][d] with row s = frame input of (session, frame) for the
    listed slots, zeros elsewhere; returns (numpy rows in slot order, device tensor)."""
    S, d = cfg["max_slots"], cfg["d_model"]
    x = np.zeros((S, d), dtype=np.float32)
    for s, sess in slot_session.items():
        x[s] = synth.frame_input(cfg, sess, slot_frame[s])
    xt = torch.from_numpy(x).to("cuda", dtype=act_torch(cfg))
    return x, xt


def rel_err_rows(y, r):
    """max over rows of ||y - r||_inf / ||r||_inf."""
    y = np.asarray(y, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    num = np.max(np.abs(y - r), axis=-1)
    den = np.maximum(np.max(np.abs(r), axis=-1), 1e-30)
    return float(np.max(num / den))


def rel_err_elem(y, r):
    """max over elements of |y - r| / max(|r|, 1e-2 ||r_row||_inf): the
    elementwise companion of rel_err_rows."""
    y = np.asarray(y, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    floor = 1e-2 * np.max(np.abs(r), axis=-1, keepdims=True)
    return float(np.max(np.abs(y - r) / np.maximum(np.abs(r), np.maximum(floor, 1e-30))))


def to_np(t):
    return t.float().cpu().numpy()


def check(cond, msg: str) -> None:
    """Assertion without pytest's expansion of large arrays in the report."""
    if not bool(cond):
        raise AssertionError(msg)
