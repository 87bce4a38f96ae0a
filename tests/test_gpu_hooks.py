"""The measurement and test hooks on the GPU: the attention kernel's
device-clock trace (fd_trace_attention), the per-kind launch timing
(fd_profile) and the persistent walk's forced abort (fd_walk_abort_next).
The first two may not change what a step computes; after the third the
ctx must recover to the undisturbed result."""
import os

import numpy as np
import pytest
import torch

import synth
from frame_decode_amd.abi import FD_E_DEVICE, FD_E_INVAL, FD_E_STATE, FD_E_UNSUPPORTED, FdError
from tests.helpers import check, make_context, rows_input, say

pytestmark = pytest.mark.gpu


def _ctx(cfg, tune=None):
    model = synth.Model(cfg, gain_noise=True)
    if tune:
        os.environ["FD_TUNE"] = tune
    try:
        return make_context(cfg, model)
    finally:
        if tune:
            del os.environ["FD_TUNE"]


def test_attention_trace_stamps_every_task_and_changes_nothing():
    """Two chunks of 256 positions per (slot, kv head), one free slot,
    sessions at frames 0, 70 and 300: the traced step's outputs, cache and
    positions equal the untraced step's bit for bit; every task of the
    traced layer writes four non-decreasing stamps (a task with no work:
    three equal exit stamps; the tasks run the slots longest window
    first); bad arguments are refused."""
    cfg = synth.scaled_config("7b_s8_p256", n_layers=3, d_model=512, n_heads=4, n_kv_heads=4,
                              d_ffn=1024, max_slots=4, max_context=512)
    say("trace: bf16/FP8, 4 slots, 2 chunks")
    ctx = _ctx(cfg, tune="attn.chunks=2")
    slots = ctx.fd_alloc_slots(3)
    start = dict(zip(slots, [0, 70, 300]))
    sess = {s: 500 + s for s in slots}
    for s in slots:
        if start[s]:
            for l in range(cfg["n_layers"]):
                v = synth.prefill_values(cfg, sess[s], l, start[s])
                ctx.fd_kv_write(s, l, 0, torch.from_numpy(v).cuda())
            ctx.fd_set_position(s, start[s])
    _, x = rows_input(cfg, sess, start)
    tasks = cfg["max_slots"] * cfg["n_kv_heads"] * 2
    y0 = torch.empty((cfg["max_slots"], cfg["d_model"]), device="cuda", dtype=torch.bfloat16)
    y1 = torch.empty_like(y0)

    ctx.fd_step(x, y0)
    ctx.fd_sync()
    arena0 = ctx.arena_view().clone()
    for s in slots:
        ctx.fd_set_position(s, start[s])

    stamps = torch.zeros((tasks, 4), device="cuda", dtype=torch.int64)
    ctx.fd_trace_attention(stamps, layer=1)
    ctx.fd_step(x, y1)
    ctx.fd_sync()
    ctx.fd_trace_attention(None)
    check(torch.equal(y0, y1), "the traced step's outputs differ")
    check(torch.equal(arena0, ctx.arena_view()), "the traced step's cache differs")
    for s in slots:
        assert ctx.fd_slot_state(s) == (1, start[s] + 1)

    st = stamps.cpu().numpy()
    check(bool(np.all(st != 0)), "a task wrote no stamp")
    check(bool(np.all(np.diff(st, axis=1) >= 0)), "stamps go backwards")
    span_us = (st[:, 3].max() - st[:, 0].min()) / 100.0
    check(0 < span_us < 1e5, f"span {span_us} us")
    # workgroup (r, head, chunk) runs slot order[r]: the active slots by
    # descending position (ties by slot), then the free one; it has work
    # when its slot is active and the chunk starts below the slot's p + 1
    # attended positions
    order = sorted(slots, key=lambda s: (-start[s], s)) + [s for s in range(cfg["max_slots"])
                                                        if s not in slots]
    idle = [((r * cfg["n_kv_heads"] + g) * 2 + c) for r, s in enumerate(order)
            for g in range(cfg["n_kv_heads"]) for c in range(2)
            if s not in slots or c * 256 >= start[s] + 1]
    check(len(idle) == 4 * 2 + 2 * 4, f"{len(idle)} idle tasks")
    check(bool(np.all(st[idle, 1] == st[idle, 3])), "an idle task timed a stream")
    busy = sorted(set(range(tasks)) - set(idle))
    check(bool(np.all(st[busy, 2] > st[busy, 1])), "a working task streamed in no time")
    say(f"trace: span {span_us:.1f} us over {tasks} tasks")

    # off: a later step leaves the buffer alone
    stamps.zero_()
    for s in slots:
        ctx.fd_set_position(s, start[s])
    ctx.fd_step(x, y1)
    ctx.fd_sync()
    check(int(stamps.abs().sum().item()) == 0, "stamps written while off")

    small = torch.zeros((tasks - 1, 4), device="cuda", dtype=torch.int64)
    for args, why in (((small, 0), "short buffer"), ((stamps, cfg["n_layers"]), "layer out of range"),
                      ((stamps, -1), "negative layer")):
        with pytest.raises(FdError) as e:
            ctx.fd_trace_attention(*args)
        assert e.value.status == FD_E_INVAL, why
    ctx.fd_destroy()


def test_attention_trace_refused_by_the_walk():
    cfg = synth.scaled_config("7b_s8_p256", n_layers=2, d_model=256, n_heads=2, n_kv_heads=2,
                              d_ffn=512, max_slots=4, max_context=64, exec_mode=1)
    ctx = _ctx(cfg)
    stamps = torch.zeros((64, 4), device="cuda", dtype=torch.int64)
    with pytest.raises(FdError) as e:
        ctx.fd_trace_attention(stamps, layer=0)
    assert e.value.status == FD_E_UNSUPPORTED
    ctx.fd_destroy()


def test_walk_abort_path_marks_slots_stale_and_recovers():
    """The persistent walk's bounded-wait abort path, forced from the host
    (fd_walk_abort_next: the launch starts with its abort flag set, so every
    workgroup leaves at its first barrier wait and nothing waits out a
    timeout): fd_sync reports FD_E_DEVICE, fd_step then refuses the stale
    slots with FD_E_STATE, and after fd_set_position the step gives the
    outputs, cache and positions of an undisturbed context bit for bit.
    The kernel-sequence profile refuses the hook."""
    cfg = synth.scaled_config("7b_s8_p256", n_layers=2, d_model=256, n_heads=2, n_kv_heads=2,
                              d_ffn=512, max_slots=4, max_context=64, exec_mode=1)
    say("walk abort: two contexts")
    a = _ctx(cfg)
    b = _ctx(cfg)
    sa, sb = a.fd_alloc_slots(3), b.fd_alloc_slots(3)
    assert sa == sb == [0, 1, 2]
    for ctx in (a, b):  # (the arenas start uninitialised: compare them from zero)
        ctx.arena_view().zero_()
    torch.cuda.synchronize()
    sess = {s: 700 + s for s in sa}
    frames = {s: 0 for s in sa}
    _, x = rows_input(cfg, sess, frames)
    ya = torch.empty((cfg["max_slots"], cfg["d_model"]), device="cuda", dtype=torch.bfloat16)
    yb = torch.empty_like(ya)
    for ctx, y in ((a, ya), (b, yb)):  # one normal step on both
        ctx.fd_step(x, y)
        ctx.fd_sync()
    frames = {s: 1 for s in sa}
    _, x = rows_input(cfg, sess, frames)

    a.fd_walk_abort_next()
    a.fd_step(x, ya)
    with pytest.raises(FdError) as e:
        a.fd_sync()
    assert e.value.status == FD_E_DEVICE
    with pytest.raises(FdError) as e:
        a.fd_step(x, ya)
    assert e.value.status == FD_E_STATE
    for s in sa:
        a.fd_set_position(s, 1)
    a.fd_step(x, ya)
    a.fd_sync()
    b.fd_step(x, yb)
    b.fd_sync()
    check(torch.equal(ya, yb), "the recovered step's outputs differ from an undisturbed step's")
    check(torch.equal(a.arena_view(), b.arena_view()), "the recovered step's cache differs")
    for s in sa:
        assert a.fd_slot_state(s) == b.fd_slot_state(s) == (1, 2)
    a.fd_destroy()
    b.fd_destroy()

    k = _ctx(dict(cfg, exec_mode=0))
    with pytest.raises(FdError) as e:
        k.fd_walk_abort_next()
    assert e.value.status == FD_E_UNSUPPORTED
    k.fd_destroy()


def test_profile_kinds_split_the_depth_stack():
    """Talker geometry with a 2-step, 2-layer depth loop: the main stack's
    projections and attention count one launch per layer (plus a reduce
    where the plan splits K), the depth stack's under their own kinds, one
    per depth step and layer."""
    cfg = synth.scaled_config("talker_s56", n_layers=3, d_model=384, d_ffn=768, max_slots=5,
                              max_context=64, depth_steps=2, depth_layers=2, depth_d=256,
                              depth_heads=2, depth_kv_heads=2, depth_ffn=512)
    ctx = _ctx(cfg)
    slots = ctx.fd_alloc_slots(3)
    _, x = rows_input(cfg, {s: 10 + s for s in slots}, {s: 0 for s in slots})
    y = torch.empty((cfg["max_slots"], cfg["d_model"]), device="cuda", dtype=torch.float32)
    d = torch.empty((cfg["max_slots"], 2, 256), device="cuda", dtype=torch.float32)
    ctx.fd_profile(True)
    ctx.fd_profile_read()
    ctx.fd_step(x, y, d)
    k = ctx.fd_profile_read()
    ctx.fd_profile(False)
    say(f"profile kinds: { {n: v[1] for n, v in k.items() if v[1]} }")
    L, DL = cfg["n_layers"], 2 * 2
    for name in ("qkv", "attention", "o_proj", "gate_up", "down"):
        check(L <= k[name][1] <= 3 * L, f"{name}: {k[name][1]} launches for {L} layers")
        check(DL <= k["depth_" + name][1] <= 3 * DL, f"depth_{name}: {k['depth_' + name][1]} launches")
        check(k[name][0] > 0 and k["depth_" + name][0] > 0, f"{name}: no time")
    check(k["attention"][1] % L == 0 and k["depth_attention"][1] % DL == 0, "attention launch counts")
    assert k["depth_in"][1] == 1 and k["walk"][1] == 0
    ctx.fd_destroy()
