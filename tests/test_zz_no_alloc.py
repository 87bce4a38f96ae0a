"""fd_step_static -- the decode step on the library's static device scratch,
for callers that cannot allocate -- against fd_step, through the C ABI.

Each profile runs on two contexts built from the same weights and cache
contents: one steps with fd_step (its fd_init workspace), the other with
fd_step_static.  The kernels and launch shapes are the same, so outputs,
cache bytes and positions must be bit-identical (stricter than the 2e-2 /
1e-3 parity bars).  Calls alternate between a larger bf16/FP8 profile and a
smaller fp32 profile with the depth loop, so each call starts from the
scratch the other profile left behind.  Profiles the scratch cannot serve
are refused with no launch."""
import numpy as np
import pytest
import torch

import synth
from frame_decode_amd.abi import FD_E_UNSUPPORTED, FD_STATIC_SCRATCH_BYTES, FdError
from tests.helpers import check, make_context, rows_input, say

pytestmark = pytest.mark.gpu


def _profile_a():
    # 7B head geometry (MHA 128-dim heads, bf16 weights, FP8 cache) at
    # reduced width and depth, 40 slots (3 m-tiles), 5 sessions active
    cfg = synth.scaled_config("7b_s8_p256", n_layers=2, d_model=512, n_heads=4, n_kv_heads=4,
                              d_ffn=1024, max_slots=40, max_context=128)
    return cfg, [0, 5, 64, 126, 33]


def _profile_b():
    # talker geometry (fp32, GQA 4:1, 256-dim heads) with the 8-step depth
    # loop, whose per-frame cache also lives in the scratch; 5 slots
    cfg = synth.scaled_config("talker_s56", n_layers=2, d_model=384, d_ffn=768, max_slots=5,
                              max_context=64, depth_layers=2, depth_d=256, depth_heads=2,
                              depth_kv_heads=2, depth_ffn=512)
    return cfg, [0, 17, 62]


class _Twin:
    """Two contexts of one profile with identical weights, cache and slots."""

    def __init__(self, cfg, start):
        self.cfg = cfg
        model = synth.Model(cfg)
        self.ref = make_context(cfg, model)
        self.sta = make_context(cfg, model)
        # cache bytes never written stay equal too
        self.ref.arena.zero_()
        self.sta.arena.zero_()
        self.slots = self.ref.fd_alloc_slots(len(start))
        check(self.sta.fd_alloc_slots(len(start)) == self.slots, "same slot ids")
        self.sess = {s: 300 + s for s in self.slots}
        self.pos = dict(zip(self.slots, start))
        for s, p in self.pos.items():
            if p:
                for l in range(cfg["n_layers"]):
                    v = torch.from_numpy(synth.prefill_values(cfg, self.sess[s], l, p)).cuda()
                    self.ref.fd_kv_write(s, l, 0, v)
                    self.sta.fd_kv_write(s, l, 0, v)
                self.ref.fd_set_position(s, p)
                self.sta.fd_set_position(s, p)
        torch.cuda.synchronize()
        dt = torch.bfloat16 if cfg["act_dtype"] == "bf16" else torch.float32
        S = cfg["max_slots"]
        self.y = [torch.empty((S, cfg["d_model"]), device="cuda", dtype=dt) for _ in range(2)]
        self.z = None
        if cfg.get("depth_steps", 0):
            self.z = [torch.empty((S, cfg["depth_steps"], cfg["depth_d"]), device="cuda", dtype=dt)
                      for _ in range(2)]

    def step(self, tag):
        cfg = self.cfg
        _, x = rows_input(cfg, self.sess, dict(self.pos))
        for t in self.y:
            t.fill_(3.0)
        if self.z is not None:
            for t in self.z:
                t.fill_(3.0)
        self.ref.fd_step(x, self.y[0], self.z[0] if self.z else None)
        self.sta.fd_step_static(x, self.y[1], self.z[1] if self.z else None)
        self.ref.fd_sync()
        self.sta.fd_sync()
        check(torch.equal(self.y[0], self.y[1]), f"{tag}: y_out differs from fd_step's")
        if self.z is not None:
            check(torch.equal(self.z[0], self.z[1]), f"{tag}: depth_out differs from fd_step's")
        check(torch.equal(self.ref.arena, self.sta.arena), f"{tag}: cache bytes differ")
        for s in self.slots:
            check(self.ref.fd_slot_state(s) == self.sta.fd_slot_state(s), f"{tag}: slot {s} state")
        act = sorted(self.slots)
        yv = self.y[1].float().cpu().numpy()
        check(np.all(np.isfinite(yv[act])), f"{tag}: non-finite outputs")
        inactive = [s for s in range(cfg["max_slots"]) if s not in act]
        check(np.all(yv[inactive] == 0), f"{tag}: inactive rows must be zero")
        say(f"  {tag}: bit-identical to fd_step (rows {act}, positions {[self.pos[s] for s in act]})")
        for s in self.slots:
            self.pos[s] += 1


def test_static_scratch_step_matches_fd_step_twice_in_a_row():
    """Two calls in a row (the second on a smaller profile and input), then
    the pair again: each bit-identical to fd_step on its twin context."""
    say("no-alloc: build the larger bf16/FP8 profile")
    a = _Twin(*_profile_a())
    say("no-alloc: build the smaller fp32 profile with the depth loop")
    b = _Twin(*_profile_b())
    check(a.ref.sizes["workspace"] > b.ref.sizes["workspace"], "profile b is the smaller one")
    check(a.ref.sizes["workspace"] <= FD_STATIC_SCRATCH_BYTES, "profile a fits the scratch")
    a.step("call 1 (bf16/FP8, 40 slots)")
    b.step("call 2 (fp32 + depth loop, 5 slots)")
    a.step("call 3 (bf16/FP8 again)")
    b.step("call 4 (fp32 again)")


def test_static_scratch_refuses_what_it_cannot_hold():
    """A walk profile and a profile whose workspace exceeds the scratch are
    refused with FD_E_UNSUPPORTED; nothing is launched and no position moves."""
    cases = [
        ("walk", synth.scaled_config("tiny", max_slots=2, exec_mode=1)),
        # no layers, 2048 slots of width 4096 in fp32: the residual stream
        # alone is 32 MiB, beyond the scratch with the other buffers
        ("oversized", synth.scaled_config("tiny", n_layers=0, d_model=4096, n_heads=32, n_kv_heads=32,
                                          head_dim=128, d_ffn=4096, max_slots=2048, max_context=4)),
    ]
    for tag, cfg in cases:
        say(f"no-alloc refusal: {tag}")
        model = synth.Model(cfg)
        ctx = make_context(cfg, model)
        if tag == "oversized":
            check(ctx.sizes["workspace"] > FD_STATIC_SCRATCH_BYTES, "profile exceeds the scratch")
        slots = ctx.fd_alloc_slots(2)
        x = torch.zeros((cfg["max_slots"], cfg["d_model"]), device="cuda")
        y = torch.full((cfg["max_slots"], cfg["d_model"]), 5.0, device="cuda")
        with pytest.raises(FdError) as ei:
            ctx.fd_step_static(x, y)
        check(ei.value.status == FD_E_UNSUPPORTED, f"{tag}: status {ei.value.status}")
        ctx.fd_sync()
        check(bool(torch.all(y == 5.0)), f"{tag}: y_out written")
        for s in slots:
            check(ctx.fd_slot_state(s) == (1, 0), f"{tag}: position moved")
        ctx.fd_destroy()
