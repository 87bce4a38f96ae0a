"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (same plan, same kernels, all slots stepped together).

Sessions are independent: a session's output depends only on its own
inputs and cache (the oracle's isolation invariant, checked bit-exactly on
the GPU by test_gpu_parity).  So where the host cannot hold every session's
cache, the GPU runs every slot and the oracle recomputes a seeded sample of
sessions one by one; the other slots carry device-drawn cache contents of
the same distribution and are checked for what holds at any size (finite
output rows, zero rows for inactive slots, positions advancing).

Tolerances: max relative row error 2e-2 on the bf16 / FP8 path, 1e-3 on the
fp32 path (the talker workload, depth outputs included).
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import synth
from oracle import Oracle, fp8
from tests.helpers import act_torch, check, make_context, rel_err_elem, rel_err_rows, say, to_np

pytestmark = pytest.mark.gpu

_POOL = ThreadPoolExecutor(max_workers=8)


@pytest.fixture(scope="module")
def model7b():
    """Weights of the 7B stack (identical for every 7B workload: they depend
    on the layer shapes only)."""
    cfg = synth.get_config("7b_s8_p256")
    say("fullsize: generating 7B weights")
    m = synth.Model(cfg)
    list(_POOL.map(m.layer, range(cfg["n_layers"])))
    yield m
    m.close()


def _prefill_host(ctx, orc, cfg, slot, session, n):
    """Positions 0..n-1 of every layer from the seeded generator, on both sides."""
    if n == 0:
        return
    vals = list(_POOL.map(lambda l: synth.prefill_values(cfg, session, l, n), range(cfg["n_layers"])))
    for l, v in enumerate(vals):
        orc.prefill(slot, l, v)
        ctx.fd_kv_write(slot, l, 0, torch.from_numpy(v).cuda())


def _prefill_device(ctx, cfg, slots, n_of, seed):
    """Device-drawn cache contents (same distribution) for slots the oracle
    does not recompute."""
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    nmax = max([n_of[s] for s in slots] + [1])
    src = torch.randn((2, cfg["n_kv_heads"], nmax, cfg["head_dim"]), generator=gen, device="cuda")
    src.mul_(synth.kv_std(cfg))
    for s in slots:
        n = n_of[s]
        if n:
            v = src[:, :, :n].contiguous()
            for l in range(cfg["n_layers"]):
                ctx.fd_kv_write(s, l, 0, v)
    torch.cuda.synchronize()


def _inputs(cfg, sess, frame):
    """x_in with the frame input of (session, frame) in each active slot."""
    S, d = cfg["max_slots"], cfg["d_model"]
    x = np.zeros((S, d), dtype=np.float32)
    for s, q in sess.items():
        x[s] = synth.frame_input(cfg, q, frame[s])
    return x, torch.from_numpy(x).to("cuda", dtype=act_torch(cfg))


def _step(ctx, cfg, sess, pos):
    x_np, x = _inputs(cfg, sess, pos)
    y = torch.full((cfg["max_slots"], cfg["d_model"]), 7.0, device="cuda", dtype=act_torch(cfg))
    dout = None
    if cfg.get("depth_steps", 0):
        dout = torch.full((cfg["max_slots"], cfg["depth_steps"], cfg["depth_d"]), 7.0,
                          device="cuda", dtype=y.dtype)
    ctx.fd_step(x, y, dout)
    ctx.fd_sync()
    return x_np, to_np(y), (to_np(dout) if dout is not None else None)


def _check_rows(cfg, yg, active):
    inactive = [s for s in range(cfg["max_slots"]) if s not in active]
    check(np.all(yg[inactive] == 0), "rows of inactive slots must be zero")
    check(np.all(np.isfinite(yg[sorted(active)])), "active rows must be finite")


def _check_new_codes(ctx, orc, cfg, slots, pos):
    """The entries a step appended for the sampled sessions: FP8 codes as
    the oracle's up to the projection's rounding (almost all identical,
    decoded values within a rounding band)."""
    if cfg["kv_dtype"] != "fp8":
        return
    arena = ctx.arena_view()
    for s in slots:
        p = pos[s]
        got = arena[s, :, :, :, p, :].cpu().numpy()
        ref = orc.cache.slot(s)[:, :, :, p, :]
        same = float(np.mean(got == ref))
        vg = fp8.decode(got).astype(np.float64)
        vr = fp8.decode(ref).astype(np.float64)
        scale = np.max(np.abs(vr), axis=-1, keepdims=True)
        bad = float(np.max(np.abs(vg - vr) / (0.13 * np.abs(vr) + 0.02 * scale)))
        say(f"  slot {s} new entry: identical codes {same:.3f}, worst scaled diff {bad:.3f}")
        check(same > 0.8 and bad <= 1.0, f"slot {s}: appended codes differ from the oracle's")


# every projection on the row-split variant, at full 7B shapes: k-split
# planes (QKV), its own residual epilogue (O, no k-split), k-split partials
# with the gate/up and residual epilogues, two k-halves
ROW_SPLIT_7B = ("qkv.NG=12,qkv.P=2,qkv.KH=2,o.NG=8,o.P=1,gu.NG=12,gu.P=2,gu.KH=2,"
                "down.NG=12,down.P=11,down.KH=2")


@pytest.mark.parametrize("exec_mode,tune,proj_in",
                         [(0, None, "auto"), (1, None, "auto"), (0, None, "bf16x2"), (1, None, "bf16x2"),
                          (0, ROW_SPLIT_7B, "bf16x2")],
                         ids=["kernels", "walk", "kernels_bf16x2", "walk_bf16x2", "row_split"])
def test_7b_eight_sessions_at_position_256(model7b, exec_mode, tune, proj_in, monkeypatch):
    """The 8-session workload in full: 32 layers, every session's cache
    prefilled to 256 positions, new frame at index 256; every row checked
    (kernel sequence and persistent walk, each with fp16 and with two-part
    bf16 projection inputs, and the kernel sequence with every projection
    on the row-split variant)."""
    if tune:
        monkeypatch.setenv("FD_TUNE", tune)
    cfg = synth.get_config("7b_s8_p256")
    cfg["exec_mode"] = exec_mode
    cfg["proj_in"] = proj_in
    p0 = cfg["position"]
    say("C2: context")
    ctx = make_context(cfg, model7b)
    orc = Oracle(cfg, model7b)
    slots = ctx.fd_alloc_slots(cfg["max_slots"])
    sess = {s: 1000 + s for s in slots}
    pos = {s: p0 for s in slots}
    for s in slots:
        _prefill_host(ctx, orc, cfg, s, sess[s], p0)
        ctx.fd_set_position(s, p0)
    say("C2: step")
    x_np, yg, _ = _step(ctx, cfg, sess, pos)
    say("C2: oracle")
    ref = orc.step(slots, x_np[slots], [pos[s] for s in slots])
    e = rel_err_rows(yg[slots], ref)
    say(f"C2: max rel err {e:.3e} (elementwise {rel_err_elem(yg[slots], ref):.3e})")
    assert e <= 2e-2
    _check_rows(cfg, yg, set(slots))
    _check_new_codes(ctx, orc, cfg, slots, pos)
    for s in slots:
        assert ctx.fd_slot_state(s) == (1, p0 + 1)
    ctx.fd_destroy()


@pytest.mark.parametrize("exec_mode", [0, 1], ids=["kernels", "walk"])
def test_7b_eighty_sessions_full_window_sampled(model7b, exec_mode):
    """80 sessions at the full 1500-frame window (new frame at index 1499):
    every slot stepped, three seeded sessions recomputed by the oracle
    (kernel sequence and persistent walk)."""
    cfg = synth.get_config("7b_s80_p1499")
    cfg["exec_mode"] = exec_mode
    p0 = cfg["position"]
    say("C3: context")
    ctx = make_context(cfg, model7b)
    orc = Oracle(cfg, model7b)
    slots = ctx.fd_alloc_slots(cfg["max_slots"])
    rng = np.random.default_rng(11)
    sample = sorted(int(s) for s in rng.choice(slots, size=3, replace=False))
    sess = {s: 2000 + s for s in slots}
    pos = {s: p0 for s in slots}
    say(f"C3: prefill (sampled slots {sample})")
    for s in sample:
        _prefill_host(ctx, orc, cfg, s, sess[s], p0)
    _prefill_device(ctx, cfg, [s for s in slots if s not in sample], pos, seed=5)
    for s in slots:
        ctx.fd_set_position(s, p0)
    say("C3: step")
    x_np, yg, _ = _step(ctx, cfg, sess, pos)
    _check_rows(cfg, yg, set(slots))
    say("C3: oracle")
    ref = orc.step(sample, x_np[sample], [p0] * len(sample))
    e = rel_err_rows(yg[sample], ref)
    say(f"C3: max rel err {e:.3e} (elementwise {rel_err_elem(yg[sample], ref):.3e})")
    assert e <= 2e-2
    _check_new_codes(ctx, orc, cfg, sample, pos)
    # the full window is reached: a further step must be refused
    from frame_decode_amd import FdError
    with pytest.raises(FdError):
        _step(ctx, cfg, sess, {s: p0 + 1 for s in slots})
    ctx.fd_destroy()


# A session with a short history is ill-conditioned on the 7B stack with an
# FP8 cache: with few positions the attention output is (nearly) the
# quantised value of the new entry itself, so a rounding difference anywhere
# upstream flips FP8 codes and the flips compound over 32 layers.  Measured
# with the oracle alone on a new session (position 0): its float32 and
# float64 evaluations differ by 1.6e-2, and a 1e-5 relative perturbation of
# the input moves the output by 3.9e-2; at position 20 the float32/float64
# gap is 7.5e-4.  Sessions below SHORT positions are therefore compared with
# the float64 oracle, and the GPU must be within the tolerance, or as close
# to it as the float32 oracle is (within a factor 3), or as close as the
# float64 oracle with its projection inputs rounded to bf16 (the activation
# type the PersonaPlex page names, "Compressing the Temporal KV cache"): no
# less precise than the method at its stated precision.
SHORT = 16


@pytest.mark.parametrize("exec_mode,proj_in", [(0, "auto"), (0, "bf16x2"), (1, "auto")],
                         ids=["kernels", "kernels_bf16x2", "walk"])
def test_7b_ragged_with_admission_and_retirement(model7b, exec_mode, proj_in):
    """The ragged workload: 56 of 80 slots active with seeded lengths
    L_i ~ U{1..1500}, new frame at L_i - 1; then sessions that reached the
    window are retired, new sessions are admitted into the lowest free
    slots at position 0 and one sampled session is freed, over three steps
    with an unchanged launch (kernel sequence, and the whole step as one
    persistent walk; projection inputs in fp16 and as two bf16 parts).
    Sampled sessions (shortest, longest, one in between, and the admitted
    ones) are recomputed by the oracle; a short session's margin under its
    bound (bound / error) and the elementwise error are printed."""
    cfg = synth.get_config("7b_ragged_80x56")
    cfg["exec_mode"] = exec_mode
    cfg["proj_in"] = proj_in
    S = cfg["max_slots"]
    say("C4: context")
    ctx = make_context(cfg, model7b)
    orc = Oracle(cfg, model7b)
    orc64 = Oracle(cfg, model7b, dtype=np.float64)  # sessions with short histories
    orcb = Oracle(cfg, model7b, dtype=np.float64, act_round="bf16")  # (the pages' activation type)
    act, lengths = synth.ragged_slots(cfg, cfg["n_active"])
    got = ctx.fd_alloc_slots(S)
    assert got == list(range(S))
    ctx.fd_free([s for s in range(S) if s not in set(act.tolist())])
    L = dict(zip(act.tolist(), lengths.tolist()))
    pos = {s: L[s] - 1 for s in L}
    sess = {s: 3000 + s for s in L}
    order = sorted(L, key=lambda s: L[s])
    sample = sorted({order[0], order[len(order) // 2], order[-1]})
    say(f"C4: prefill (sampled slots {sample}, lengths {[L[s] for s in sample]})")
    for s in sample:
        _prefill_host(ctx, orc, cfg, s, sess[s], pos[s])
        if pos[s] < SHORT:
            for l in range(cfg["n_layers"]):
                orc64.prefill(s, l, synth.prefill_values(cfg, sess[s], l, pos[s]))
                orcb.prefill(s, l, synth.prefill_values(cfg, sess[s], l, pos[s]))
    _prefill_device(ctx, cfg, [s for s in L if s not in sample], pos, seed=6)
    for s in L:
        ctx.fd_set_position(s, pos[s])
    tracked = list(sample)
    next_sess = 4000
    for step in range(3):
        active = set(sess)
        say(f"C4: step {step}: {len(active)} active, tracked {[(s, pos[s]) for s in tracked]}")
        x_np, yg, _ = _step(ctx, cfg, sess, pos)
        _check_rows(cfg, yg, active)
        ref = orc.step(tracked, x_np[tracked], [pos[s] for s in tracked])
        short = [s for s in tracked if pos[s] < SHORT]
        ref64, refb = {}, {}
        if short:
            r64 = orc64.step(short, x_np[short], [pos[s] for s in short])
            ref64 = dict(zip(short, r64))
            refb = dict(zip(short, orcb.step(short, x_np[short], [pos[s] for s in short])))
        for i, s in enumerate(tracked):
            e = rel_err_rows(yg[s][None], ref[i][None])
            ee = rel_err_elem(yg[s][None], ref[i][None])
            if s in ref64:
                e64 = rel_err_rows(yg[s][None], ref64[s][None])
                cond = rel_err_rows(ref[i][None], ref64[s][None])
                cond_b = rel_err_rows(refb[s][None], ref64[s][None])
                # no farther from the exact step than 3x the float32 oracle,
                # or than the step at the pages' own activation type (bf16)
                bound = max(2e-2, 3.0 * cond, cond_b)
                say(f"  slot {s} (position {pos[s]}): vs float32 oracle {e:.3e} (elementwise {ee:.3e}), "
                    f"vs float64 {e64:.3e}, float32 oracle vs float64 {cond:.3e}, "
                    f"bf16-activation oracle vs float64 {cond_b:.3e}, bound {bound:.3e}, "
                    f"margin {bound / max(e64, 1e-30):.2f}x")
                assert e64 <= bound, f"step {step} slot {s}"
            else:
                say(f"  slot {s} (position {pos[s]}): rel err {e:.3e} (elementwise {ee:.3e})")
                assert e <= 2e-2, f"step {step} slot {s}: {e}"
        _check_new_codes(ctx, orc, cfg, [s for s in tracked if pos[s] >= SHORT], pos)
        for s in active:
            pos[s] += 1
            assert ctx.fd_slot_state(s) == (1, pos[s])
        # retire sessions whose window is full, free one tracked session,
        # admit two new ones (lowest free slots, position 0)
        full = [s for s in active if pos[s] >= cfg["max_context"]]
        drop = [tracked[0]] if step == 0 else []
        gone = sorted(set(full) | set(drop))
        if gone:
            ctx.fd_free(gone)
        for s in gone:
            del sess[s], pos[s]
            if s in tracked:
                tracked.remove(s)
        free_before = sorted(set(range(S)) - set(sess))
        new = ctx.fd_alloc_slots(2)
        assert new == free_before[:2], "admission takes the lowest free slots"
        for s in new:
            sess[s] = next_sess
            next_sess += 1
            pos[s] = 0
            orc.cache.kv.pop(s, None)  # a new session starts from an empty cache
            orc64.cache.kv.pop(s, None)
            orcb.cache.kv.pop(s, None)
            assert ctx.fd_slot_state(s) == (1, 0)
        tracked = sorted(tracked + new)
    ctx.fd_destroy()


@pytest.mark.parametrize("exec_mode", [0, 1], ids=["kernels", "walk"])
def test_talker_fifty_six_sessions_with_depth_loop_sampled(exec_mode):
    """The talker workload in full (26-layer fp32 main stack with GQA 4:1 and
    head_dim 256, 56 sessions at index 1499, then the 8-step depth loop of
    the 6-layer depth stack, as separate launches or the whole step as one
    persistent walk): two seeded sessions recomputed, 1e-3 on the main
    output and on all eight depth outputs."""
    cfg = synth.get_config("talker_s56")
    cfg["exec_mode"] = exec_mode
    p0 = cfg["position"]
    say("C5: weights")
    model = synth.Model(cfg)
    list(_POOL.map(model.layer, range(cfg["n_layers"])))
    list(_POOL.map(model.depth_layer, range(cfg["depth_layers"])))
    say("C5: context")
    ctx = make_context(cfg, model)
    orc = Oracle(cfg, model)
    slots = ctx.fd_alloc_slots(cfg["max_slots"])
    rng = np.random.default_rng(12)
    sample = sorted(int(s) for s in rng.choice(slots, size=2, replace=False))
    sess = {s: 5000 + s for s in slots}
    pos = {s: p0 for s in slots}
    say(f"C5: prefill (sampled slots {sample})")
    for s in sample:
        _prefill_host(ctx, orc, cfg, s, sess[s], p0)
    _prefill_device(ctx, cfg, [s for s in slots if s not in sample], pos, seed=7)
    for s in slots:
        ctx.fd_set_position(s, p0)
    say("C5: step")
    x_np, yg, zg = _step(ctx, cfg, sess, pos)
    _check_rows(cfg, yg, set(slots))
    check(np.all(np.isfinite(zg)), "depth outputs must be finite")
    say("C5: oracle")
    ref, zref = orc.step(sample, x_np[sample], [p0] * len(sample))
    e = rel_err_rows(yg[sample], ref)
    ez = rel_err_rows(zg[sample].reshape(-1, cfg["depth_d"]), zref.reshape(-1, cfg["depth_d"]))
    say(f"C5: max rel err {e:.3e}, depth {ez:.3e}")
    assert e <= 1e-3 and ez <= 1e-3
    ctx.fd_destroy()
    model.close()
