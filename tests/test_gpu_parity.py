"""GPU parity of the HIP decode step against the oracle, through the C ABI,
at sizes the oracle finishes in seconds (several tiles, ragged tails,
multi-chunk attention).  Tolerances: max relative row error 1e-3 on the
fp32 path, 2e-2 on the bf16/FP8 path; cache indexing bit-exact."""
import os

import numpy as np
import pytest
import torch

import synth
from oracle import Oracle, fp8
from tests.helpers import check, make_context, rel_err_elem, rel_err_rows, rows_input, say, to_np

pytestmark = pytest.mark.gpu


def _sentinel_fill(ctx, cfg):
    if cfg["kv_dtype"] == "fp8":
        ctx.arena.fill_(0x7F)
    else:
        ctx.arena.view(torch.int32)[: ctx.arena.numel() // 4].fill_(0x7FC00001)
    torch.cuda.synchronize()


def _is_sentinel(a: np.ndarray, fp8_cache: bool) -> np.ndarray:
    if fp8_cache:
        return a == 0x7F
    return a.view(np.int32) == 0x7FC00001


def test_encoder_bit_exact_and_layout():
    """fd_kv_write stores code(value / sigma) exactly as the oracle's codec,
    at the documented offsets; special values included."""
    cfg = synth.scaled_config("7b_s8_p256", n_layers=2, d_model=256, n_heads=2, n_kv_heads=2,
                              d_ffn=256, max_slots=3, max_context=64)
    model = synth.Model(cfg)
    say("encoder: build ctx")
    ctx = make_context(cfg, model)
    _sentinel_fill(ctx, cfg)
    rng = np.random.default_rng(3)
    n = 40
    vals = (rng.standard_normal((2, 2, n, 128)) * 3.0).astype(np.float32)
    sig = model.kv_scale[1]  # [2][H_kv]
    # exact ties between codes, values beyond 448 * sigma, tiny subnormals
    codes_all = fp8.DECODE_TABLE[np.isfinite(fp8.DECODE_TABLE)]
    mids = (np.sort(np.unique(np.abs(codes_all)))[:-1] + np.sort(np.unique(np.abs(codes_all)))[1:]) / 2
    k = min(128, mids.size)
    vals[0, 0, 1, :k] = (mids[:k] * sig[0, 0]).astype(np.float32)
    vals[0, 1, 2, :8] = np.array([500, -500, 1e6, -1e-30, 0, -0.0, 448, 449], np.float32) * sig[0, 1]
    src = torch.from_numpy(vals).cuda()
    ctx.fd_kv_write(1, 1, 5, src)
    torch.cuda.synchronize()
    arena = ctx.arena_view().cpu().numpy()
    got = arena[1, 1, :, :, 5:5 + n, :]
    expect = fp8.encode(vals / sig.astype(np.float32)[:, :, None, None])
    # -0.0 / sigma keeps its sign; the oracle codec returns 0x80 for it
    check(np.array_equal(got, expect), "np.array_equal(got, expect)")
    mask = np.ones(arena.shape, dtype=bool)
    mask[1, 1, :, :, 5:5 + n, :] = False
    check(np.all(arena[mask] == 0x7F), "bytes outside the written range changed")


def _run_steps(cfg, model, slot_pos, n_steps, *, tol, sentinel=True, gain_noise=False):
    """Prefill each listed slot to its start position, then step n_steps
    frames; compare every step's outputs with the oracle."""
    say(f"parity: cfg L={cfg['n_layers']} d={cfg['d_model']} S={cfg['max_slots']} "
        f"kv={cfg['kv_dtype']} slots={slot_pos}")
    ctx = make_context(cfg, model)
    if sentinel:
        _sentinel_fill(ctx, cfg)
    orc = Oracle(cfg, model)
    slots = ctx.fd_alloc_slots(len(slot_pos))
    sess = {s: 100 + s for s in slots}
    pos = dict(zip(slots, slot_pos))
    for s in slots:
        p = pos[s]
        if p:
            for l in range(cfg["n_layers"]):
                v = synth.prefill_values(cfg, sess[s], l, p)
                orc.prefill(s, l, v)
                ctx.fd_kv_write(s, l, 0, torch.from_numpy(v).cuda())
            ctx.fd_set_position(s, p)
    worst = 0.0
    y = torch.empty((cfg["max_slots"], cfg["d_model"]), device="cuda",
                    dtype=torch.bfloat16 if cfg["act_dtype"] == "bf16" else torch.float32)
    dout = None
    if cfg.get("depth_steps", 0):
        dout = torch.empty((cfg["max_slots"], cfg["depth_steps"], cfg["depth_d"]), device="cuda",
                           dtype=y.dtype)
    for step in range(n_steps):
        x_np, x = rows_input(cfg, sess, {s: pos[s] for s in slots})
        y.fill_(7.0)
        ctx.fd_step(x, y, dout)
        ctx.fd_sync()
        act = sorted(slots)
        ref = orc.step(act, x_np[act], [pos[s] for s in act])
        if dout is not None:
            ref, zref = ref
        yg = to_np(y)
        e = rel_err_rows(yg[act], ref)
        worst = max(worst, e)
        say(f"  step {step}: max rel err {e:.3e}")
        assert e <= tol, f"step {step}: {e}"
        inactive = [s for s in range(cfg["max_slots"]) if s not in act]
        check(np.all(yg[inactive] == 0), "inactive rows must be zero")
        if dout is not None:
            zg = to_np(dout)
            ez = rel_err_rows(zg[act].reshape(-1, cfg["depth_d"]), zref.reshape(-1, cfg["depth_d"]))
            say(f"  depth: max rel err {ez:.3e}")
            assert ez <= tol
            check(np.all(zg[inactive] == 0), "np.all(zg[inactive] == 0)")
        for s in slots:
            pos[s] += 1
            assert ctx.fd_slot_state(s) == (1, pos[s])
    dev = ctx.slot_table_view().cpu().numpy()
    for s in slots:
        assert dev[1, s] == pos[s], "device position must advance with the host's"
    # attention order: a permutation, the active slots first by descending
    # position (ties by slot), then the inactive ones ascending
    order = [int(v) for v in dev[2]]
    S = cfg["max_slots"]
    want = sorted(slots, key=lambda s: (-pos[s], s)) + [s for s in range(S) if s not in slots]
    check(order == want, f"attention order {order[:8]}... differs from {want[:8]}...")
    return ctx, orc, slots, pos, worst


def _check_cache(ctx, orc, cfg, slots, pos, start):
    """Cache bytes: written exactly at positions start[s]..pos[s]-1 (plus the
    prefill), never elsewhere; values equal the oracle's up to the rounding
    of the projection (FP8: codes within one step, almost all identical)."""
    fp8_cache = cfg["kv_dtype"] == "fp8"
    arena = ctx.arena_view().cpu().numpy()
    for s in range(cfg["max_slots"]):
        a = arena[s]
        if s not in slots:
            untouched = bool(np.all(_is_sentinel(a, fp8_cache)))
            assert untouched, f"slot {s} touched"
            continue
        p = pos[s]
        hole = bool(np.any(_is_sentinel(a[:, :, :, :p, :], fp8_cache)))
        past = bool(np.all(_is_sentinel(a[:, :, :, p:, :], fp8_cache)))
        assert not hole, f"slot {s}: unwritten entry below position {p}"
        assert past, f"slot {s}: write at or past position {p}"
        ref = orc.cache.slot(s)[:, :, :, :p, :]
        got = a[:, :, :, :p, :]
        new = slice(start[s], p)
        if fp8_cache:
            # prefilled entries were encoded from identical fp32 values: bit-exact
            pre_ok = bool(np.array_equal(got[:, :, :, :start[s]], ref[:, :, :, :start[s]]))
            assert pre_ok, f"slot {s}: prefilled codes differ"
            g = got[:, :, :, new]
            r = ref[:, :, :, new]
            same = float(np.mean(g == r))
            # decoded values: the new entries come from bf16 activations on
            # the GPU and fp32 ones in the oracle, so they agree to within
            # the projection's rounding (relative to each head vector)
            vg = fp8.decode(g).astype(np.float64)
            vr = fp8.decode(r).astype(np.float64)
            scale = np.max(np.abs(vr), axis=-1, keepdims=True)
            bad = float(np.max(np.abs(vg - vr) / (0.13 * np.abs(vr) + 0.02 * scale)))
            ok = same > 0.8 and bad <= 1.0
            assert ok, f"slot {s}: identical codes {same:.3f}, worst scaled diff {bad:.3f}"
        else:
            err = float(np.max(np.abs(got - ref)) / np.max(np.abs(ref)))
            assert err < 1e-4, f"slot {s}: cache values differ by {err:.3e}"


@pytest.mark.parametrize("exec_mode", [0, 1], ids=["kernels", "walk"])
def test_tiny_fp32_sixteen_frames(exec_mode):
    """Two sessions x 16 frames from an empty fp32 cache (the tiny
    workload), 1e-3, with the cache checked byte-for-byte against the
    sentinel fill; as a kernel sequence and as one persistent walk."""
    cfg = synth.get_config("tiny")
    cfg["exec_mode"] = exec_mode
    model = synth.Model(cfg, gain_noise=True)
    ctx, orc, slots, pos, worst = _run_steps(cfg, model, [0, 0], 16, tol=1e-3)
    _check_cache(ctx, orc, cfg, slots, pos, {s: 0 for s in slots})


@pytest.mark.parametrize("exec_mode,proj_in", [(0, "auto"), (0, "bf16x2"), (1, "auto"), (1, "bf16x2")],
                         ids=["kernels", "kernels_bf16x2", "walk", "walk_bf16x2"])
def test_bf16_fp8_ragged_multichunk(exec_mode, proj_in):
    """bf16 weights/activations, FP8 cache, 7B head geometry (128-dim MHA)
    at reduced width and depth; slots at positions spanning 1..3 attention
    chunks, one slot left empty; kernel sequence and persistent walk, each
    with the projection inputs in fp16 and as two bf16 parts."""
    cfg = synth.scaled_config("7b_s8_p256", n_layers=3, d_model=512, n_heads=4, n_kv_heads=4,
                              d_ffn=1536, max_slots=9, max_context=700, exec_mode=exec_mode,
                              proj_in=proj_in)
    model = synth.Model(cfg, gain_noise=True)
    start = [0, 1, 239, 240, 241, 300, 480, 690]
    # this window is short enough for one chunk by default: ask the plan
    # for three (it rounds chunks up to whole wave loads of 8 positions:
    # 240, 240, 220) so the chunk merge is exercised; frames 240 and 480
    # open a chunk holding only the new entry
    os.environ["FD_TUNE"] = "attn.chunks=3"
    try:
        ctx, orc, slots, pos, worst = _run_steps(cfg, model, start, 3, tol=2e-2)
    finally:
        del os.environ["FD_TUNE"]
    _check_cache(ctx, orc, cfg, slots, pos, dict(zip(slots, start)))


# every path of the row-split projection variant: k-split planes (QKV),
# its own epilogue without k-splits (O with one k-half, down with two and a
# ragged last n-group: residual, next norm input), k-split partials through
# the reduce kernel with the gate/up epilogue
ROW_SPLIT_TUNE = ("qkv.NG=12,qkv.P=2,qkv.KH=2,o.NG=8,o.P=1,o.KH=1,gu.NG=16,gu.P=2,gu.KH=2,"
                  "down.NG=12,down.P=1,down.KH=2")


@pytest.mark.parametrize("max_slots,proj_in", [(9, "bf16x2"), (40, "bf16x2"), (9, "f16"), (40, "f16")])
def test_row_split_projections(max_slots, proj_in):
    """The row-split projection variant (two-part or fp16 rows; its waves own
    different weight rows and share the activations through LDS; one or two
    k-halves) on
    every projection of a reduced 7B-geometry bf16/FP8 stack, with one and
    with three 16-row tiles of sessions: 2e-2, cache indexing bit-exact."""
    cfg = synth.scaled_config("7b_s8_p256", n_layers=2, d_model=512, n_heads=4, n_kv_heads=4,
                              d_ffn=1536, max_slots=max_slots, max_context=300, proj_in=proj_in)
    model = synth.Model(cfg, gain_noise=True)
    start = [(37 * i) % 290 for i in range(max_slots - 2)]
    os.environ["FD_TUNE"] = ROW_SPLIT_TUNE
    try:
        ctx, orc, slots, pos, worst = _run_steps(cfg, model, start, 3, tol=2e-2)
    finally:
        del os.environ["FD_TUNE"]
    _check_cache(ctx, orc, cfg, slots, pos, dict(zip(slots, start)))


@pytest.mark.parametrize("exec_mode", [0, 1], ids=["kernels", "walk"])
def test_fp32_gqa_with_depth_loop(exec_mode):
    """Talker geometry (GQA 4:1, head_dim 256, fp32) at reduced width, with
    the 8-step depth loop of a 128-dim-head stack (as separate launches and
    as one persistent walk of the whole step); 1e-3."""
    cfg = synth.scaled_config("talker_s56", n_layers=2, d_model=384, d_ffn=768, max_slots=5,
                              max_context=300, depth_layers=2, depth_d=256, depth_heads=2,
                              depth_kv_heads=2, depth_ffn=512, exec_mode=exec_mode)
    model = synth.Model(cfg, gain_noise=True)
    start = [0, 63, 64, 200]
    ctx, orc, slots, pos, worst = _run_steps(cfg, model, start, 2, tol=1e-3)
    _check_cache(ctx, orc, cfg, slots, pos, dict(zip(slots, start)))


@pytest.mark.parametrize("max_slots,x3", [(40, 0), (70, 0), (5, 1), (56, 1), (90, 1)],
                         ids=["f32-3tiles", "f32-5tiles", "x3-1tile", "x3-4tiles", "x3-6tiles"])
def test_fp32_projection_tilings(max_slots, x3):
    """fp32 projections of the talker geometry (with its depth loop and
    input projection) at several 16-row tilings of sessions: with fp32
    products at three and five tiles (the one- and two-block kernels with
    and without k-splits, planes, reduce and direct epilogues), and with the
    opt-in three-product loop (FD_TUNE x3=1: weights and rows as bf16 high
    and low parts, w_lo*x_hi + w_hi*x_lo + w_hi*x_hi with fp32 sums) at one,
    four and (two m-groups of at most five) six tiles: 1e-3, cache indexing
    bit-exact."""
    cfg = synth.scaled_config("talker_s56", n_layers=2, d_model=384, d_ffn=768, max_slots=max_slots,
                              max_context=300, depth_layers=2, depth_d=256, depth_heads=2,
                              depth_kv_heads=2, depth_ffn=512, exec_mode=0)
    model = synth.Model(cfg, gain_noise=True)
    start = [0, 63, 64, 200] if max_slots == 5 else [(37 * i) % 290 for i in range(max_slots - 2)]
    if x3:
        os.environ["FD_TUNE"] = "x3=1"
    try:
        ctx, orc, slots, pos, worst = _run_steps(cfg, model, start, 2, tol=1e-3)
    finally:
        os.environ.pop("FD_TUNE", None)
    _check_cache(ctx, orc, cfg, slots, pos, dict(zip(slots, start)))


def test_admission_and_free_keep_launch_shape():
    """Sessions freed and admitted between steps: new sessions start at
    position 0 in the lowest free slot, equal a fresh oracle session, and
    the other sessions are unaffected (bit-identical to an undisturbed run)."""
    cfg = synth.scaled_config("7b_s8_p256", n_layers=2, d_model=256, n_heads=2, n_kv_heads=2,
                              d_ffn=512, max_slots=4, max_context=64)
    model = synth.Model(cfg)
    say("admission: two contexts")
    a = make_context(cfg, model)
    b = make_context(cfg, model)
    sa = a.fd_alloc_slots(3)
    sb = b.fd_alloc_slots(3)
    assert sa == sb == [0, 1, 2]
    y_a = torch.empty((4, 256), device="cuda", dtype=torch.bfloat16)
    y_b = torch.empty_like(y_a)
    sess = {0: 10, 1: 11, 2: 12}
    frames = {0: 0, 1: 0, 2: 0}
    for t in range(3):
        _, x = rows_input(cfg, sess, frames)
        a.fd_step(x, y_a)
        b.fd_step(x, y_b)
        for s in frames:
            frames[s] += 1
    # in b: end session 1 and admit a new one (goes to slot 1, position 0)
    b.fd_free([1])
    assert b.fd_alloc_slots(1) == [1]
    assert b.fd_slot_state(1) == (1, 0)
    sess_b = dict(sess)
    sess_b[1] = 99
    frames_b = dict(frames)
    frames_b[1] = 0
    orc = Oracle(cfg, model)
    for t in range(4):
        _, xa = rows_input(cfg, sess, frames)
        xb_np, xb = rows_input(cfg, sess_b, frames_b)
        a.fd_step(xa, y_a)
        b.fd_step(xb, y_b)
        torch.cuda.synchronize()
        ya, yb = to_np(y_a), to_np(y_b)
        check(np.array_equal(ya[[0, 2]], yb[[0, 2]]), "other sessions must be bit-identical")
        ref = orc.step([1], xb_np[[1]], [frames_b[1]])
        assert rel_err_rows(yb[[1]], ref) <= 2e-2
        for s in frames:
            frames[s] += 1
            frames_b[s] += 1


@pytest.mark.parametrize("exec_mode", [0, 1], ids=["kernels", "walk"])
def test_deterministic_and_isolated(exec_mode):
    """Two runs give bit-identical outputs; changing other slots' inputs
    and caches leaves a session's output bit-identical (both modes)."""
    cfg = synth.scaled_config("7b_s8_p256", n_layers=2, d_model=512, n_heads=4, n_kv_heads=4,
                              d_ffn=1024, max_slots=6, max_context=400, exec_mode=exec_mode)
    model = synth.Model(cfg)
    say("determinism: ctx")
    ctx = make_context(cfg, model)
    slots = ctx.fd_alloc_slots(6)
    for s in slots:
        for l in range(cfg["n_layers"]):
            ctx.fd_kv_write(s, l, 0, torch.from_numpy(synth.prefill_values(cfg, s, l, 350)).cuda())
    outs = []
    for run in range(3):
        for s in slots:
            ctx.fd_set_position(s, 350)
        sess = {s: s for s in slots}
        _, x = rows_input(cfg, sess, {s: 350 for s in slots})
        if run == 2:  # perturb slots 0 and 5: inputs and caches
            x[0] = torch.randn_like(x[0]) * 5
            x[5] = 0
            ctx.arena_view()[0].random_(0, 127)
            ctx.arena_view()[5].random_(0, 127)
        y = torch.empty_like(x)
        ctx.fd_step(x, y)
        ctx.fd_sync()
        outs.append(to_np(y))
    check(np.array_equal(outs[0], outs[1]), "np.array_equal(outs[0], outs[1])")
    check(np.array_equal(outs[0][1:5], outs[2][1:5]), "np.array_equal(outs[0][1:5], outs[2][1:5])")


@pytest.mark.parametrize("proj_in", ["f16", "bf16x2"])
def test_row_beyond_fp16_range_stays_in_its_session(proj_in):
    """A session whose frame is scaled by 1e6 (finite in bf16, beyond fp16's
    65504 once it is a projection input): with fp16 rows its own output row
    is non-finite, with two bf16 parts it is finite; either way every other
    session's row is bit-identical to the run without it."""
    cfg = synth.scaled_config("7b_s8_p256", n_layers=2, d_model=512, n_heads=4, n_kv_heads=4,
                              d_ffn=1024, max_slots=6, max_context=400, proj_in=proj_in)
    model = synth.Model(cfg, gain_noise=True)
    say(f"fp16 range: {proj_in}")
    ctx = make_context(cfg, model)
    slots = ctx.fd_alloc_slots(6)
    for s in slots:
        for l in range(cfg["n_layers"]):
            ctx.fd_kv_write(s, l, 0, torch.from_numpy(synth.prefill_values(cfg, s, l, 350)).cuda())
    outs = []
    for big in (False, True):
        for s in slots:
            ctx.fd_set_position(s, 350)
        _, x = rows_input(cfg, {s: s for s in slots}, {s: 350 for s in slots})
        if big:
            x[2] = x[2] * 1e6
        y = torch.empty_like(x)
        ctx.fd_step(x, y)
        ctx.fd_sync()
        outs.append(to_np(y))
    rest = [s for s in slots if s != 2]
    check(np.array_equal(outs[0][rest], outs[1][rest]), "another session's row changed")
    check(bool(np.all(np.isfinite(outs[0]))), "the plain run must be finite")
    finite = bool(np.all(np.isfinite(outs[1][2])))
    check(finite == (proj_in == "bf16x2"), f"scaled session finite: {finite}")
    ctx.fd_destroy()


def _prefill_rolling(ctx, orc, cfg, s, session, p):
    """Fill the window before frame p (frames max(0, p-T+1)..p-1) with
    seeded values: the oracle at their absolute frame indices, the GPU at
    cache positions (frame mod T) through its own encoder."""
    T = cfg["max_context"]
    n = min(p, T - 1)
    f0 = p - n
    for l in range(cfg["n_layers"]):
        v = synth.prefill_values(cfg, session, l, n)
        orc.prefill(s, l, v, t0=f0)
        i = 0
        while i < n:
            c0 = (f0 + i) % T
            run = min(n - i, T - c0)
            ctx.fd_kv_write(s, l, c0, torch.from_numpy(np.ascontiguousarray(v[:, :, i:i + run])).cuda())
            i += run
    ctx.fd_set_position(s, p)


@pytest.mark.parametrize("exec_mode", [0, 1], ids=["kernels", "walk"])
@pytest.mark.parametrize("family", ["fp32", "bf16_fp8"])
def test_rolling_window_across_the_wrap(family, exec_mode):
    """Rolling window (kv_ring = 1): sessions before, at and well past the
    window length step across the wrap of their cache positions; outputs
    match the oracle (which keeps frames by absolute index) every step, and
    each new entry lands at cache position (frame mod T)."""
    if family == "fp32":
        cfg = synth.scaled_config("tiny", max_slots=6, max_context=64, kv_ring=1, exec_mode=exec_mode)
        start, tol, tune = [0, 61, 63, 64, 130, 200], 1e-3, None
    else:
        cfg = synth.scaled_config("7b_s8_p256", n_layers=2, d_model=512, n_heads=4, n_kv_heads=4,
                                  d_ffn=1024, max_slots=6, max_context=1100, kv_ring=1,
                                  exec_mode=exec_mode)
        # three chunks of the window (368, 368, 364 positions): the new
        # entry's position falls in different chunks as the frame advances
        start, tol, tune = [0, 1097, 1099, 1100, 1655, 3000], 2e-2, "attn.chunks=3"
    T = cfg["max_context"]
    model = synth.Model(cfg, gain_noise=True)
    say(f"rolling window: {family} {'walk' if exec_mode else 'kernels'} T={T} start={start}")
    if tune:
        os.environ["FD_TUNE"] = tune
    try:
        ctx = make_context(cfg, model)
    finally:
        if tune:
            del os.environ["FD_TUNE"]
    orc = Oracle(cfg, model)
    slots = ctx.fd_alloc_slots(len(start))
    sess = {s: 300 + s for s in slots}
    pos = dict(zip(slots, start))
    for s in slots:
        if pos[s]:
            _prefill_rolling(ctx, orc, cfg, s, sess[s], pos[s])
    y = torch.empty((cfg["max_slots"], cfg["d_model"]), device="cuda",
                    dtype=torch.bfloat16 if cfg["act_dtype"] == "bf16" else torch.float32)
    for step in range(4):
        x_np, x = rows_input(cfg, sess, {s: pos[s] for s in slots})
        ctx.fd_step(x, y)
        ctx.fd_sync()
        ref = orc.step(slots, x_np[slots], [pos[s] for s in slots])
        e = rel_err_rows(to_np(y)[slots], ref)
        say(f"  step {step} positions {[pos[s] for s in slots]}: max rel err {e:.3e}")
        assert e <= tol, f"step {step}: {e}"
        # the new entries: cache position p mod T holds frame p (layer 1, keys and values)
        arena = ctx.arena_view().cpu().numpy()
        for s in slots:
            p = pos[s]
            got = arena[s, 1, :, :, p % T, :]
            want = orc.cache.slot(s)[1, :, :, p, :]
            if cfg["kv_dtype"] == "fp8":
                same = float(np.mean(got == want))
                check(same > 0.8, f"slot {s} frame {p}: only {same:.3f} of the codes agree")
            else:
                err = float(np.max(np.abs(got - want)) / np.max(np.abs(want)))
                check(err < 1e-4, f"slot {s} frame {p}: new entry differs by {err:.3e}")
        for s in slots:
            pos[s] += 1
            assert ctx.fd_slot_state(s) == (1, pos[s])
    ctx.fd_destroy()


@pytest.mark.parametrize("exec_mode", [0, 1], ids=["kernels", "walk"])
@pytest.mark.parametrize("family", ["fp32", "bf16_fp8"])
def test_output_head_greedy_tokens(family, exec_mode):
    """fd_step_tokens: logits of every active slot match the oracle's head
    on the oracle's output; each token is the argmax of the GPU's own logits
    (first maximum, bit-exact) and equals the oracle's token unless the two
    are within the measured logit error of each other (a near tie); inactive
    slots give token -1 and zero logits."""
    if family == "fp32":
        cfg = synth.scaled_config("tiny", max_slots=3, vocab=512, exec_mode=exec_mode)
        start, tol = [0, 7], 1e-3
    else:
        cfg = synth.scaled_config("7b_s8_p256", n_layers=2, d_model=512, n_heads=4, n_kv_heads=4,
                                  d_ffn=1024, max_slots=6, max_context=300, vocab=2048,
                                  exec_mode=exec_mode)
        start, tol = [0, 5, 100, 255, 256], 2e-2
    model = synth.Model(cfg, gain_noise=True)
    say(f"head: {family} {'walk' if exec_mode else 'kernels'} V={cfg['vocab']}")
    ctx = make_context(cfg, model)
    orc = Oracle(cfg, model)
    slots = ctx.fd_alloc_slots(len(start))
    sess = {s: 400 + s for s in slots}
    pos = dict(zip(slots, start))
    for s in slots:
        if pos[s]:
            for l in range(cfg["n_layers"]):
                v = synth.prefill_values(cfg, sess[s], l, pos[s])
                orc.prefill(s, l, v)
                ctx.fd_kv_write(s, l, 0, torch.from_numpy(v).cuda())
            ctx.fd_set_position(s, pos[s])
    S, V = cfg["max_slots"], cfg["vocab"]
    y = torch.empty((S, cfg["d_model"]), device="cuda",
                    dtype=torch.bfloat16 if cfg["act_dtype"] == "bf16" else torch.float32)
    tokens = torch.full((S,), 12345, device="cuda", dtype=torch.int32)
    logits = torch.full((S, V), 7.0, device="cuda", dtype=torch.float32)
    inactive = [s for s in range(S) if s not in slots]
    for step in range(2):
        x_np, x = rows_input(cfg, sess, {s: pos[s] for s in slots})
        ctx.fd_step_tokens(x, y, tokens, logits if step == 0 else None)
        ctx.fd_sync()
        yref = orc.step(slots, x_np[slots], [pos[s] for s in slots])
        lref, tref = orc.head(yref)
        tg = tokens.cpu().numpy()
        check(np.all(tg[inactive] == -1), "inactive slots must give token -1")
        if step == 0:
            lg = logits.cpu().numpy()
            e = rel_err_rows(lg[slots], lref)
            say(f"  step {step}: logits max rel err {e:.3e}")
            assert e <= tol
            check(np.all(lg[inactive] == 0), "inactive slots must give zero logits")
            for i, s in enumerate(slots):
                check(tg[s] == int(np.argmax(lg[s])), f"slot {s}: token is not the first maximum of its logits")
                if tg[s] != tref[i]:
                    gap = float(lref[i].max() - lref[i][tg[s]])
                    err = float(np.max(np.abs(lg[s] - lref[i])))
                    say(f"  slot {s}: token {tg[s]} vs {tref[i]} (gap {gap:.3e}, logit error {err:.3e})")
                    check(gap <= 2 * err + 1e-6, f"slot {s}: token {tg[s]} is not a near-tie of {tref[i]}")
        else:
            agree = float(np.mean(tg[slots] == tref))
            say(f"  step {step}: tokens agree on {agree:.2f} of the sessions")
            check(agree >= 0.6, "tokens (without a logits buffer) disagree with the oracle")
        for s in slots:
            pos[s] += 1
    ctx.fd_destroy()


@pytest.mark.parametrize("proj_in", ["f16", "bf16x2"])
def test_fp8_weights_with_per_row_scales(proj_in):
    """FP8 E4M3 weights quantised by the library from bf16 sources (one
    scale per output row), bf16 activations (projection inputs in fp16, or
    as two bf16 parts), FP8 cache, with the output head: outputs and logits
    match the oracle running the dequantised weights (2e-2) over three
    steps; tokens are the first maximum of the GPU's logits."""
    cfg = synth.scaled_config("7b_s8_p256", n_layers=3, d_model=512, n_heads=4, n_kv_heads=4,
                              d_ffn=1536, max_slots=7, max_context=400, vocab=1024,
                              w_dtype="fp8", act_dtype="bf16", proj_in=proj_in)
    model = synth.Model(cfg, gain_noise=True)
    start = [0, 1, 100, 255, 256, 390]
    say(f"fp8 weights: slots {start}")
    ctx = make_context(cfg, model)
    orc = Oracle(cfg, model)
    slots = ctx.fd_alloc_slots(len(start))
    sess = {s: 500 + s for s in slots}
    pos = dict(zip(slots, start))
    for s in slots:
        if pos[s]:
            for l in range(cfg["n_layers"]):
                v = synth.prefill_values(cfg, sess[s], l, pos[s])
                orc.prefill(s, l, v)
                ctx.fd_kv_write(s, l, 0, torch.from_numpy(v).cuda())
            ctx.fd_set_position(s, pos[s])
    S, V = cfg["max_slots"], cfg["vocab"]
    y = torch.empty((S, cfg["d_model"]), device="cuda", dtype=torch.bfloat16)
    tokens = torch.empty((S,), device="cuda", dtype=torch.int32)
    logits = torch.empty((S, V), device="cuda", dtype=torch.float32)
    for step in range(3):
        x_np, x = rows_input(cfg, sess, {s: pos[s] for s in slots})
        ctx.fd_step_tokens(x, y, tokens, logits)
        ctx.fd_sync()
        ref = orc.step(slots, x_np[slots], [pos[s] for s in slots])
        lref, _ = orc.head(ref)
        e = rel_err_rows(to_np(y)[slots], ref)
        lg = logits.cpu().numpy()
        el = rel_err_rows(lg[slots], lref)
        say(f"  step {step}: output max rel err {e:.3e}, logits {el:.3e}")
        assert e <= 2e-2 and el <= 2e-2
        tg = tokens.cpu().numpy()
        for s in slots:
            check(tg[s] == int(np.argmax(lg[s])), f"slot {s}: token is not the first maximum")
        check(tg[S - 1] == -1, "the inactive slot's token must be -1")
        for s in slots:
            pos[s] += 1
    ctx.fd_destroy()


# every projection split over K, with 4- and with 6-block workgroups
FP8_SPLITS = {
    "ng6": "qkv.NG=6,qkv.P=2,o.NG=6,o.P=4,gu.NG=6,gu.P=2,down.NG=6,down.P=4",
    "ng4": "qkv.NG=4,qkv.P=4,o.NG=4,o.P=2,gu.NG=4,gu.P=4,down.NG=4,down.P=8",
}


@pytest.mark.parametrize("split,proj_in", [("ng4", "auto"), ("ng6", "auto"), ("ng6", "bf16x2")])
def test_fp8_weights_eighty_slots(split, proj_in, monkeypatch):
    """FP8 weights at 80 slots: five 16-row tiles per m-group (the kernels
    the 80-session FP8-weight step runs), 7B head geometry (MHA, 128-dim
    heads) at reduced width and depth, every projection split over K (QKV
    planes, k-split partial sums with the residual and gate/up epilogues),
    with the output head.  All 80 sessions at positions 0..150 against the
    oracle running the dequantised weights: outputs and logits 2e-2
    (projection inputs in fp16, and as two bf16 parts)."""
    monkeypatch.setenv("FD_TUNE", FP8_SPLITS[split])
    cfg = synth.scaled_config("7b_s8_p256", n_layers=2, d_model=1024, n_heads=8, n_kv_heads=8,
                              d_ffn=2048, max_slots=80, max_context=160, vocab=512,
                              w_dtype="fp8", act_dtype="bf16", proj_in=proj_in)
    model = synth.Model(cfg, gain_noise=True)
    say(f"fp8 weights, 80 slots, splits {FP8_SPLITS[split]}")
    ctx = make_context(cfg, model)
    orc = Oracle(cfg, model)
    slots = ctx.fd_alloc_slots(80)
    rng = np.random.default_rng(21)
    start = rng.integers(0, 151, size=80)
    start[:4] = [0, 1, 150, 2]
    sess = {s: 700 + s for s in slots}
    pos = {s: int(p) for s, p in zip(slots, start)}
    for s in slots:
        if pos[s]:
            for l in range(cfg["n_layers"]):
                v = synth.prefill_values(cfg, sess[s], l, pos[s])
                orc.prefill(s, l, v)
                ctx.fd_kv_write(s, l, 0, torch.from_numpy(v).cuda())
            ctx.fd_set_position(s, pos[s])
    S, V = cfg["max_slots"], cfg["vocab"]
    y = torch.empty((S, cfg["d_model"]), device="cuda", dtype=torch.bfloat16)
    tokens = torch.empty((S,), device="cuda", dtype=torch.int32)
    logits = torch.empty((S, V), device="cuda", dtype=torch.float32)
    for step in range(2):
        x_np, x = rows_input(cfg, sess, {s: pos[s] for s in slots})
        ctx.fd_step_tokens(x, y, tokens, logits)
        ctx.fd_sync()
        ref = orc.step(slots, x_np[slots], [pos[s] for s in slots])
        lref, _ = orc.head(ref)
        yg, lg = to_np(y), logits.cpu().numpy()
        e, el = rel_err_rows(yg[slots], ref), rel_err_rows(lg[slots], lref)
        say(f"  step {step}: output max rel err {e:.3e} (elementwise {rel_err_elem(yg[slots], ref):.3e}), "
            f"logits {el:.3e}")
        assert e <= 2e-2 and el <= 2e-2
        tg = tokens.cpu().numpy()
        for s in slots:
            check(tg[s] == int(np.argmax(lg[s])), f"slot {s}: token is not the first maximum")
        for s in slots:
            pos[s] += 1
    ctx.fd_destroy()


def test_misaligned_output_is_refused_without_effect():
    """A y_out that is not 16-byte aligned: FD_E_INVAL, no launch, no cache
    byte or position changed."""
    from frame_decode_amd import FdError
    from frame_decode_amd.abi import FD_E_INVAL
    cfg = synth.scaled_config("7b_s8_p256", n_layers=2, d_model=256, n_heads=2, n_kv_heads=2,
                              d_ffn=256, max_slots=4, max_context=32)
    model = synth.Model(cfg)
    ctx = make_context(cfg, model)
    _sentinel_fill(ctx, cfg)
    slots = ctx.fd_alloc_slots(2)
    _, x = rows_input(cfg, {s: 40 + s for s in slots}, {s: 0 for s in slots})
    buf = torch.zeros(cfg["max_slots"] * cfg["d_model"] + 8, device="cuda", dtype=torch.bfloat16)
    y_bad = buf[4:4 + cfg["max_slots"] * cfg["d_model"]].view(cfg["max_slots"], cfg["d_model"])
    check(y_bad.data_ptr() % 16 == 8, "test buffer is misaligned by 8 bytes")
    before = ctx.arena.clone()
    with pytest.raises(FdError) as ei:
        ctx.fd_step(x, y_bad)
    check(ei.value.status == FD_E_INVAL, f"status {ei.value.status}")
    x_bad = torch.zeros(cfg["max_slots"] * cfg["d_model"] + 8, device="cuda", dtype=torch.bfloat16)
    with pytest.raises(FdError):
        ctx.fd_step(x_bad[4:4 + x.numel()].view_as(x), torch.empty_like(x))
    ctx.fd_sync()
    check(torch.equal(before, ctx.arena), "cache bytes changed")
    check(bool(torch.all(buf == 0)), "the misaligned output was written")
    for s in slots:
        check(ctx.fd_slot_state(s) == (1, 0), "position moved")
    # an aligned step afterwards still runs
    y = torch.empty_like(x)
    ctx.fd_step(x, y)
    ctx.fd_sync()
    for s in slots:
        check(ctx.fd_slot_state(s) == (1, 1), "the aligned step did not advance")
    ctx.fd_destroy()


@pytest.mark.parametrize("exec_mode", [0, 1], ids=["kernels", "walk"])
def test_many_slots_row_groups(exec_mode):
    """140 slots (9 row tiles: the projections split the rows into two
    m-groups of 5 tiles) with 130 active sessions at ragged positions,
    bf16/FP8: every active row matches the oracle, inactive rows are zero."""
    cfg = synth.scaled_config("7b_s8_p256", n_layers=2, d_model=512, n_heads=4, n_kv_heads=4,
                              d_ffn=1024, max_slots=140, max_context=64, exec_mode=exec_mode)
    model = synth.Model(cfg, gain_noise=True)
    rng = np.random.default_rng(21)
    start = [int(v) for v in rng.integers(0, 60, size=130)]
    ctx, orc, slots, pos, worst = _run_steps(cfg, model, start, 2, tol=2e-2, sentinel=False)
    say(f"many slots: worst {worst:.3e}")


def test_largest_slot_counts_row_groups():
    """720 slots (45 row tiles: six m-groups of 8 tiles, the shape of the
    largest session count that fits in HBM), 700 active sessions at ragged
    positions, bf16/FP8: every active row matches the oracle, inactive rows
    are zero.  The six m-groups of each weight tile run on one XCD."""
    cfg = synth.scaled_config("7b_s8_p256", n_layers=2, d_model=512, n_heads=4, n_kv_heads=4,
                              d_ffn=1024, max_slots=720, max_context=64)
    model = synth.Model(cfg, gain_noise=True)
    rng = np.random.default_rng(23)
    start = [int(v) for v in rng.integers(0, 60, size=700)]
    ctx, orc, slots, pos, worst = _run_steps(cfg, model, start, 2, tol=2e-2, sentinel=False)
    say(f"720 slots: worst {worst:.3e}")


@pytest.mark.parametrize("exec_mode", [0, 1], ids=["kernels", "walk"])
def test_step_with_no_active_session(exec_mode):
    """A step with every slot free writes zero rows, changes no cache byte
    and no position; a session admitted afterwards starts at position 0."""
    cfg = synth.scaled_config("7b_s8_p256", n_layers=2, d_model=256, n_heads=2, n_kv_heads=2,
                              d_ffn=512, max_slots=4, max_context=64, exec_mode=exec_mode)
    model = synth.Model(cfg)
    ctx = make_context(cfg, model)
    _sentinel_fill(ctx, cfg)
    before = ctx.arena_view().cpu().numpy().copy()
    x = torch.randn((4, 256), device="cuda").to(torch.bfloat16)
    y = torch.full((4, 256), 3.0, device="cuda", dtype=torch.bfloat16)
    ctx.fd_step(x, y)
    ctx.fd_sync()
    check(bool(torch.all(y == 0)), "rows of free slots must be zero")
    check(np.array_equal(ctx.arena_view().cpu().numpy(), before), "the cache changed")
    for s in range(4):
        assert ctx.fd_slot_state(s) == (0, 0)
    assert ctx.fd_alloc_slots(1) == [0] and ctx.fd_slot_state(0) == (1, 0)
    ctx.fd_destroy()
