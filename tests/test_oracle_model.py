"""Pins of the oracle's decoder step and full recompute against things
other than themselves:

* a library-built reference (torch CPU, float64): F.rms_norm,
  F.scaled_dot_product_attention with a causal mask (GQA via enable_gqa),
  F.silu, and the rotary embedding as complex multiplication
  (x_{2i} + j x_{2i+1}) * exp(j p theta_i); FP8 storage through torch's own
  float8_e4m3fn conversion;
* incremental decode equal to the full causal recompute;
* session isolation (other slots' inputs, caches and activity do not change
  a session's output);
* closed-form special cases (empty stack, constant rows, first frame,
  zero query projection, zero gate);
* float64 and float32 oracles agreeing to 1e-5.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import synth
from oracle import Oracle, forward_full, depth_full, rope, rope_table, round_bf16, fp8
from oracle.decoder import quantize_rows


def small_cfg(**over):
    base = synth.get_config("tiny")
    base.update(over)
    return base


def rel_err(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-30))


# ---------------------------------------------------------------------------
# library-built reference


def torch_reference(cfg, model, X, *, depth=False, fp8_cache=None, window=None):
    """Full causal forward in float64 built from torch library routines
    (window: each frame attends to the last `window` frames only, given to
    scaled_dot_product_attention as an explicit boolean mask)."""
    if depth:
        L, hq, hkv, hd = (cfg["depth_layers"], cfg["depth_heads"], cfg["depth_kv_heads"],
                          cfg["depth_head_dim"])
        layer, g_final = model.depth_layer, model.depth_g_final
        fp8_cache = False
    else:
        L, hq, hkv, hd = cfg["n_layers"], cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"]
        layer, g_final = model.layer, model.g_final
        if fp8_cache is None:
            fp8_cache = cfg["kv_dtype"] == "fp8"
    eps = cfg["rms_eps"]
    x = torch.from_numpy(np.asarray(X, dtype=np.float64))
    T, d = x.shape
    i = torch.arange(hd // 2, dtype=torch.float64)
    theta = cfg["rope_base"] ** (-2.0 * i / hd)
    ang = torch.arange(T, dtype=torch.float64)[:, None] * theta[None, :]
    rot = torch.polar(torch.ones_like(ang), ang)

    def rot_rows(t):  # t [T, H, hd]
        c = torch.view_as_complex(t.reshape(T, t.shape[1], hd // 2, 2).contiguous())
        return torch.view_as_real(c * rot[:, None, :]).reshape(T, t.shape[1], hd)

    for l in range(L):
        w = {k: torch.from_numpy(np.asarray(v, dtype=np.float64)) for k, v in layer(l).items()}
        a = F.rms_norm(x, (d,), weight=w["g_attn"], eps=eps)
        q = rot_rows((a @ w["wq"].T).reshape(T, hq, hd))
        k = rot_rows((a @ w["wk"].T).reshape(T, hkv, hd))
        v = (a @ w["wv"].T).reshape(T, hkv, hd)
        if fp8_cache:
            sk = torch.from_numpy(np.asarray(model.kv_scale[l, 0], dtype=np.float32))[None, :, None]
            sv = torch.from_numpy(np.asarray(model.kv_scale[l, 1], dtype=np.float32))[None, :, None]
            kq = (k.float() / sk)
            vq = (v.float() / sv)
            assert float(kq.abs().max()) < 448 and float(vq.abs().max()) < 448
            k = kq.to(torch.float8_e4m3fn).to(torch.float64) * sk.double()
            v = vq.to(torch.float8_e4m3fn).to(torch.float64) * sv.double()
        if window is None:
            o = F.scaled_dot_product_attention(q.transpose(0, 1)[None], k.transpose(0, 1)[None],
                                               v.transpose(0, 1)[None], is_causal=True,
                                               enable_gqa=(hq != hkv))
        else:
            ii = torch.arange(T)[:, None]
            jj = torch.arange(T)[None, :]
            keep = (jj <= ii) & (jj > ii - window)
            o = F.scaled_dot_product_attention(q.transpose(0, 1)[None], k.transpose(0, 1)[None],
                                               v.transpose(0, 1)[None], attn_mask=keep,
                                               enable_gqa=(hq != hkv))
        o = o[0].transpose(0, 1).reshape(T, hq * hd)
        x = x + o @ w["wo"].T
        b = F.rms_norm(x, (d,), weight=w["g_ffn"], eps=eps)
        x = x + (F.silu(b @ w["w_gate"].T) * (b @ w["w_up"].T)) @ w["w_down"].T
    g = torch.from_numpy(np.asarray(g_final, dtype=np.float64))
    return F.rms_norm(x, (d,), weight=g, eps=eps).numpy()


def frames(cfg, session, T):
    return np.stack([synth.frame_input(cfg, session, t) for t in range(T)])


@pytest.fixture(scope="module")
def tiny():
    cfg = small_cfg()
    model = synth.Model(cfg, gain_noise=True)
    return cfg, model


def test_full_matches_library_reference_fp32_cache(tiny):
    cfg, model = tiny
    X = frames(cfg, 0, 16)
    ref = torch_reference(cfg, model, X)
    got = forward_full(cfg, model, X, dtype=np.float64)
    assert rel_err(got, ref) < 1e-12


def test_full_matches_library_reference_fp8_cache():
    cfg = small_cfg(kv_dtype="fp8")
    model = synth.Model(cfg, gain_noise=True)
    X = frames(cfg, 3, 12)
    ref = torch_reference(cfg, model, X)
    got = forward_full(cfg, model, X, dtype=np.float64)
    assert rel_err(got, ref) < 1e-12


def test_full_matches_library_reference_gqa():
    cfg = small_cfg(n_heads=4, n_kv_heads=1, head_dim=32, d_model=128, d_ffn=256)
    model = synth.Model(cfg, gain_noise=True)
    X = frames(cfg, 1, 9)
    ref = torch_reference(cfg, model, X)
    got = forward_full(cfg, model, X, dtype=np.float64)
    assert rel_err(got, ref) < 1e-12


def _run_incremental(cfg, model, sessions, T, dtype):
    orc = Oracle(cfg, model, dtype=dtype)
    outs = {s: [] for s in sessions}
    for t in range(T):
        x = np.stack([synth.frame_input(cfg, s, t) for s in sessions])
        y = orc.step(sessions, x, [t] * len(sessions))
        for i, s in enumerate(sessions):
            outs[s].append(y[i])
    return {s: np.stack(v) for s, v in outs.items()}, orc


@pytest.mark.parametrize("kv", ["f32", "fp8"])
def test_incremental_equals_full_recompute(kv):
    """Check (a): 16 frames stepped one at a time equal the causal forward
    over all 16 frames, for every frame."""
    cfg = small_cfg(kv_dtype=kv)
    model = synth.Model(cfg, gain_noise=True)
    outs, _ = _run_incremental(cfg, model, [0, 1], 16, np.float64)
    for s in (0, 1):
        full = forward_full(cfg, model, frames(cfg, s, 16), dtype=np.float64)
        assert rel_err(outs[s], full) < 1e-10
        # and in float32, within the rounding budget of the step
    outs32, _ = _run_incremental(cfg, model, [0, 1], 16, np.float32)
    for s in (0, 1):
        full = forward_full(cfg, model, frames(cfg, s, 16), dtype=np.float64)
        assert rel_err(outs32[s], full) < 1e-5 if kv == "f32" else 2e-3


def test_session_isolation(tiny):
    """Check (b): perturbing other slots' inputs, caches and activity leaves
    a session's output and cache bit-identical."""
    cfg, model = tiny
    base = Oracle(cfg, model)
    pert = Oracle(cfg, model)
    rng = np.random.default_rng(5)
    # slot 1 is the session under test in both; slot 0 differs
    for t in range(6):
        x1 = synth.frame_input(cfg, 11, t)
        xa = synth.frame_input(cfg, 21, t)
        xb = (rng.standard_normal(cfg["d_model"]) * 3).astype(np.float32)
        ya = base.step([0, 1], np.stack([xa, x1]), [t, t])
        yb = pert.step([0, 1], np.stack([xb, x1]), [t, t])
        assert np.array_equal(ya[1], yb[1])
    # garbage in slot 0's cache of the perturbed run, then slot 0 inactive
    pert.cache.slot(0)[...] = rng.standard_normal(pert.cache.shape).astype(np.float32) * 1e3
    x1 = synth.frame_input(cfg, 11, 6)
    ya = base.step([0, 1], np.stack([synth.frame_input(cfg, 21, 6), x1]), [6, 6])
    yb = pert.step([1], x1[None], [6])
    # the row count differs here (2 vs 1), so the BLAS blocking may differ
    assert rel_err(yb[0], ya[1]) < 1e-6
    assert np.array_equal(base.cache.slot(1), pert.cache.slot(1)) or \
        rel_err(pert.cache.slot(1), base.cache.slot(1)) < 1e-6


def test_empty_stack_is_rmsnorm_of_input():
    cfg = small_cfg(n_layers=0)
    model = synth.Model(cfg, gain_noise=True)
    e = synth.frame_input(cfg, 0, 0)
    y = Oracle(cfg, model, dtype=np.float64).step([0], e[None], [0])[0]
    ms = np.mean(e.astype(np.float64) ** 2)
    expect = e.astype(np.float64) / np.sqrt(ms + cfg["rms_eps"]) * model.g_final.astype(np.float64)
    assert rel_err(y, expect) < 1e-14


def test_constant_row():
    cfg = small_cfg(n_layers=0)
    model = synth.Model(cfg, gain_noise=True)
    c = 0.37
    y = Oracle(cfg, model, dtype=np.float64).step([0], np.full((1, cfg["d_model"]), c), [0])[0]
    expect = model.g_final.astype(np.float64) * c / np.sqrt(c * c + cfg["rms_eps"])
    assert rel_err(y, expect) < 1e-14


def _one_layer(kv="f32", zero=()):
    cfg = small_cfg(n_layers=1, kv_dtype=kv)
    return cfg, synth.Model(cfg, gain_noise=True, zero=zero)


def test_first_frame_attends_to_itself_only():
    """p = 0: the softmax has one weight equal to 1, so the output does not
    depend on the query/key projections and attention returns V_hat_0."""
    cfg, m = _one_layer(zero=("w_gate",))
    e = synth.frame_input(cfg, 0, 0)
    y = Oracle(cfg, m, dtype=np.float64).step([0], e[None], [0])[0]
    w = m.layer(0)
    e64 = e.astype(np.float64)
    a = e64 / np.sqrt(np.mean(e64 ** 2) + cfg["rms_eps"]) * w["g_attn"]
    x = e64 + w["wo"] @ (w["wv"] @ a)
    expect = x / np.sqrt(np.mean(x ** 2) + cfg["rms_eps"]) * m.g_final
    assert rel_err(y, expect) < 1e-12
    # different q/k projections: same output
    cfg2, m2 = _one_layer(zero=("w_gate", "wq", "wk"))
    y2 = Oracle(cfg2, m2, dtype=np.float64).step([0], e[None], [0])[0]
    assert rel_err(y2, y) < 1e-13


def _torch_bf16(v):
    """bf16 rounding by torch's own conversion (float32 -> bfloat16, nearest
    even), back to float64; v must hold float32 values."""
    t = torch.from_numpy(np.asarray(v, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float64).numpy()


def test_round_bf16_is_torchs_bfloat16_conversion():
    """The oracle's bf16 rounding equals torch's float32 -> bfloat16
    conversion on random values over many binades, on exact ties (low 16
    bits 0x8000, both parities of the kept bits) and on signed zeros; from
    float64 it rounds once (1 + 2^-8 + 2^-40 lies above the tie, so it
    goes up, where rounding through float32 first would land on the tie
    and go to even)."""
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(200_000) * np.exp2(rng.integers(-40, 40, 200_000))).astype(np.float32)
    bits = rng.integers(0, 2**32, 50_000, dtype=np.uint64).astype(np.uint32)
    ties = ((bits & np.uint32(0xFFFF0000)) | np.uint32(0x8000)).view(np.float32)
    ties = ties[np.isfinite(ties) & (np.abs(ties) > 1e-37) & (np.abs(ties) < 1e37)]
    for v in (x, ties, np.array([0.0, -0.0], dtype=np.float32)):
        got = round_bf16(v).astype(np.float64)
        assert np.array_equal(got.view(np.uint64), _torch_bf16(v).view(np.uint64))
    one = np.array([1.0 + 2.0 ** -8 + 2.0 ** -40])
    assert round_bf16(one)[0] == 1.0 + 2.0 ** -7
    assert _torch_bf16(one.astype(np.float32))[0] == 1.0


def test_bf16_activations_first_frame_closed_form():
    """act_round="bf16" at p = 0 over one layer with an fp32 cache: the
    attention output is the new value vector, so the step reduces to
    a = bf(rms(e) g_attn), x = e + W_o bf(W_v a), b = bf(rms(x) g_ffn),
    y = rms(x + W_down bf(silu(W_gate b) * (W_up b))) g_final, assembled here
    in float64 with torch's bf16 conversion (the float32 stage of that
    conversion lands on no bf16 tie for these inputs).  The rounded step
    also differs from the unrounded one."""
    cfg, m = _one_layer()
    e = synth.frame_input(cfg, 0, 0)
    y = Oracle(cfg, m, dtype=np.float64, act_round="bf16").step([0], e[None], [0])[0]
    y_full = Oracle(cfg, m, dtype=np.float64).step([0], e[None], [0])[0]
    w = {k: np.asarray(v, dtype=np.float64) for k, v in m.layer(0).items()}
    eps = cfg["rms_eps"]
    ties = []

    def bf(v):
        f = v.astype(np.float32)
        ties.append(int(np.sum((f.view(np.uint32) & np.uint32(0xFFFF)) == 0x8000)))
        return _torch_bf16(f)

    def rms(v, g):
        return v / np.sqrt(np.mean(v ** 2) + eps) * g

    e64 = e.astype(np.float64)
    a = bf(rms(e64, w["g_attn"]))
    x = e64 + w["wo"] @ bf(w["wv"] @ a)
    b = bf(rms(x, w["g_ffn"]))
    g = w["w_gate"] @ b
    x = x + w["w_down"] @ bf(g / (1.0 + np.exp(-g)) * (w["w_up"] @ b))
    expect = rms(x, np.asarray(m.g_final, dtype=np.float64))
    assert sum(ties) == 0
    assert rel_err(y, expect) < 1e-12
    assert rel_err(y, y_full) > 1e-5
    with pytest.raises(ValueError):
        Oracle(cfg, m, act_round="fp16")


@pytest.mark.parametrize("kv", ["f32", "fp8"])
def test_zero_query_gives_uniform_average(kv):
    """W_q = 0: every score is 0, so attention is the plain mean of the
    cached values over positions 0..p (new frame included)."""
    cfg, m = _one_layer(kv, zero=("wq", "w_gate"))
    orc = Oracle(cfg, m, dtype=np.float64)
    p = 9
    vals = synth.prefill_values(cfg, 4, 0, p)
    orc.prefill(0, 0, vals)
    e = synth.frame_input(cfg, 4, p)
    y = orc.step([0], e[None], [p])[0]
    w = m.layer(0)
    e64 = e.astype(np.float64)
    a = e64 / np.sqrt(np.mean(e64 ** 2) + cfg["rms_eps"]) * w["g_attn"]
    vnew = (w["wv"] @ a).reshape(cfg["n_kv_heads"], cfg["head_dim"])
    V = np.concatenate([vals[1].astype(np.float64), vnew[:, None, :]], axis=1)  # [H][p+1][D]
    if kv == "fp8":
        s = m.kv_scale[0, 1].astype(np.float32)[:, None, None]
        V = fp8.decode(fp8.encode(V.astype(np.float32) / s)).astype(np.float64) * s
    o = V.mean(axis=1).reshape(-1)
    x = e64 + w["wo"] @ o
    expect = x / np.sqrt(np.mean(x ** 2) + cfg["rms_eps"]) * m.g_final
    assert rel_err(y, expect) < 1e-12


def test_zero_gate_ffn_adds_nothing():
    cfg, m = _one_layer(zero=("w_gate",))
    cfg2, m2 = _one_layer(zero=("w_gate", "w_down"))
    o1 = Oracle(cfg, m, dtype=np.float64)
    o2 = Oracle(cfg2, m2, dtype=np.float64)
    for t in range(4):
        e = synth.frame_input(cfg, 2, t)[None]
        assert np.array_equal(o1.step([0], e, [t]), o2.step([0], e, [t]))


def test_float64_and_float32_agree():
    cfg = small_cfg()
    model = synth.Model(cfg)
    o64, _ = _run_incremental(cfg, model, [0, 1], 8, np.float64)
    o32, _ = _run_incremental(cfg, model, [0, 1], 8, np.float32)
    for s in (0, 1):
        assert rel_err(o32[s], o64[s]) < 1e-5


def test_talker_shape_float64_and_float32_agree():
    cfg = small_cfg(n_layers=2, d_model=128, n_heads=4, n_kv_heads=1, head_dim=64, d_ffn=384,
                    depth_steps=3, depth_layers=2, depth_d=96, depth_heads=2, depth_kv_heads=2,
                    depth_head_dim=48, depth_ffn=160)
    model = synth.Model(cfg)
    ys = {}
    for dt in (np.float64, np.float32):
        orc = Oracle(cfg, model, dtype=dt)
        for t in range(4):
            x = np.stack([synth.frame_input(cfg, s, t) for s in (0, 1)])
            ys[dt] = orc.step([0, 1], x, [t, t])
    assert rel_err(ys[np.float32][0], ys[np.float64][0]) < 1e-5
    assert rel_err(ys[np.float32][1], ys[np.float64][1]) < 1e-5


def test_depth_loop_is_teacher_forced_causal_forward():
    """The depth loop's k-th output equals row k of a causal forward of the
    depth stack over the inputs it actually saw (c + z_{k-1}), and that
    forward equals the library-built reference."""
    cfg = small_cfg(n_layers=1, d_model=128, n_heads=4, n_kv_heads=1, head_dim=64, d_ffn=384,
                    depth_steps=8, depth_layers=2, depth_d=96, depth_heads=2, depth_kv_heads=2,
                    depth_head_dim=48, depth_ffn=160)
    model = synth.Model(cfg, gain_noise=True)
    orc = Oracle(cfg, model, dtype=np.float64)
    x = np.stack([synth.frame_input(cfg, s, 0) for s in (0, 1)])
    y, z = orc.step([0, 1], x, [0, 0])
    for i in range(2):
        c = model.w_in.astype(np.float64) @ y[i]
        inputs = np.stack([c] + [c + z[i, k] for k in range(cfg["depth_steps"] - 1)])
        full = depth_full(cfg, model, inputs, dtype=np.float64)
        assert rel_err(z[i], full) < 1e-10
        ref = torch_reference(cfg, model, inputs, depth=True)
        assert rel_err(full, ref) < 1e-12


def test_rope_pins():
    D, base = 64, 10000.0
    cos, sin = rope_table(1500, D, base, np.float64)
    rng = np.random.default_rng(0)
    q = rng.standard_normal((1, 1, D))
    k = rng.standard_normal((1, 1, D))
    # table against a float64 evaluation: within one float32 ulp
    c32, s32 = rope_table(1500, D, base, np.float32)
    assert np.all(np.abs(c32 - cos) <= np.spacing(np.abs(c32).astype(np.float32)))
    assert np.all(np.abs(s32 - sin) <= np.spacing(np.abs(s32).astype(np.float32)))
    # pair norms preserved
    for p in (0, 1, 77, 1499):
        r = rope(q, np.array([p]), cos, sin)
        assert np.allclose(np.hypot(r[..., 0::2], r[..., 1::2]),
                           np.hypot(q[..., 0::2], q[..., 1::2]), rtol=1e-13)
    # scores depend only on the offset
    for m, n, c in ((5, 3, 100), (0, 0, 1400), (1499, 10, -8)):
        a = np.sum(rope(q, np.array([m]), cos, sin) * rope(k, np.array([n]), cos, sin))
        b = np.sum(rope(q, np.array([m + c]), cos, sin) * rope(k, np.array([n + c]), cos, sin))
        assert abs(a - b) < 1e-10
    # direction: the complex-multiplication form of the same rotation
    p = 321
    zc = (q[0, 0, 0::2] + 1j * q[0, 0, 1::2]) * np.exp(1j * p * base ** (-np.arange(D // 2) * 2.0 / D))
    r = rope(q, np.array([p]), cos, sin)[0, 0]
    assert np.allclose(r[0::2], zc.real, atol=1e-12) and np.allclose(r[1::2], zc.imag, atol=1e-12)


# ---------------------------------------------------------------------------
# rolling window (sessions longer than the window)


@pytest.mark.parametrize("kv", ["f32", "fp8"])
def test_sliding_full_matches_library_reference(kv):
    """The full recompute with a 5-frame window equals torch's attention
    with an explicit sliding-window mask, over 14 frames."""
    cfg = small_cfg(kv_dtype=kv, kv_ring=1, max_context=5)
    model = synth.Model(cfg, gain_noise=True)
    X = frames(cfg, 2, 14)
    ref = torch_reference(cfg, model, X, window=5)
    got = forward_full(cfg, model, X, dtype=np.float64)
    assert rel_err(got, ref) < 1e-12
    # and the window matters: without it the late frames differ
    plain = torch_reference(cfg, model, X)
    assert rel_err(got[-1], plain[-1]) > 1e-3


@pytest.mark.parametrize("kv", ["f32", "fp8"])
def test_rolling_window_incremental_equals_sliding_recompute(kv):
    """A 6-frame rolling window stepped one frame at a time over 20 frames
    (the window wraps three times) equals the sliding-window recompute at
    every frame; rotary positions are the absolute frame indices."""
    cfg = small_cfg(kv_dtype=kv, kv_ring=1, max_context=6)
    model = synth.Model(cfg, gain_noise=True)
    outs, _ = _run_incremental(cfg, model, [0, 1], 20, np.float64)
    for s in (0, 1):
        full = forward_full(cfg, model, frames(cfg, s, 20), dtype=np.float64)
        assert rel_err(outs[s], full) < 1e-10


def test_rolling_window_before_it_fills_equals_fixed_window(tiny):
    """Until a session reaches the window length, the rolling and the fixed
    window are the same computation (bit-identical outputs)."""
    cfg, model = tiny
    ring = dict(cfg, kv_ring=1)
    a, _ = _run_incremental(cfg, model, [0, 1], cfg["max_context"] if cfg["max_context"] < 12 else 12,
                            np.float32)
    b, _ = _run_incremental(ring, model, [0, 1], cfg["max_context"] if cfg["max_context"] < 12 else 12,
                            np.float32)
    for s in (0, 1):
        assert np.array_equal(a[s], b[s])


def test_rolling_window_prefill_at_absolute_frames():
    """A session prefilled with the window's earlier frames at their absolute
    indices and stepped at frame p gives the same output as one that
    stepped through every frame (the cache only holds what the window
    reads)."""
    cfg = small_cfg(kv_ring=1, max_context=6, n_layers=1)
    model = synth.Model(cfg, gain_noise=True)
    outs, stepped = _run_incremental(cfg, model, [0], 15, np.float64)
    # rebuild frames 9..13 of session 0's cache from the stepped oracle, then step frame 14
    orc = Oracle(cfg, model, dtype=np.float64)
    hist = stepped.cache.slot(0)[:, :, :, 9:14, :]
    orc.cache.slot(3, 14)[:, :, :, 9:14, :] = hist
    y = orc.step([3], synth.frame_input(cfg, 0, 14)[None], [14])
    assert rel_err(y[0], outs[0][14]) < 1e-12


# ---------------------------------------------------------------------------
# output head (greedy token per frame)


def test_head_closed_forms_and_ties():
    """Head rows that are unit vectors pick out coordinates of y; equal
    logits resolve to the lowest token index (the token equals a plain scan
    for the largest (logit, -index)); a positive rescaling of the hidden
    state leaves the tokens unchanged."""
    cfg = small_cfg(vocab=32)
    model = synth.Model(cfg)
    orc = Oracle(cfg, model, dtype=np.float64)
    d = cfg["d_model"]
    rng = np.random.default_rng(5)
    y = rng.standard_normal((3, d))
    y[1, 7] = 50.0  # row 1: tokens 0 and 2 (both coordinate 7) tie for the maximum
    cols = [7, 3, 7] + list(range(10, 39))
    model.w_head = np.zeros((32, d))
    for v, c in enumerate(cols):
        model.w_head[v, c] = 1.0
    logits, tok = orc.head(y)
    assert np.array_equal(logits[:, 0], y[:, 7]) and np.array_equal(logits[:, 1], y[:, 3])
    assert tok[1] == 0
    for i in range(3):
        assert tok[i] == max(range(32), key=lambda v: (logits[i, v], -v))
    model.w_head = rng.standard_normal((32, d))
    _, t1 = orc.head(y)
    _, t2 = orc.head(3.5 * y)
    assert np.array_equal(t1, t2)


# ---------------------------------------------------------------------------
# FP8 weights with per-output-row scales


def test_fp8_weight_rows_pins():
    """Per-row E4M3 quantisation: each row's largest magnitude maps to the
    code of +-448 and comes back to within an fp32 ulp (the scale max/448 is
    rounded once), every entry in the normal range is within half a step
    (2^-4 relative) and in the subnormal range within 2^-10 * scale; a zero
    row stays zero with scale 1; a row scaled by 2^k keeps its codes."""
    rng = np.random.default_rng(9)
    w = (rng.standard_normal((40, 96)) * np.exp(rng.uniform(-6, 2, (40, 1)))).astype(np.float32)
    w[3] = 0.0
    w[7, 5] = -3.75  # a clear row maximum with negative sign
    wq, sc = quantize_rows(w)
    for i in range(40):
        if i == 3:
            assert sc[i] == 1.0 and not np.any(wq[i])
            continue
        j = int(np.argmax(np.abs(w[i])))
        code = int(fp8.encode(np.asarray([w[i, j] / sc[i]], np.float32))[0])
        assert code == (0xFE if w[i, j] < 0 else 0x7E)
        assert abs(float(wq[i, j]) - float(w[i, j])) <= 2.0 ** -22 * abs(float(w[i, j]))
        rel = np.abs(w[i]) / sc[i]
        normal = rel >= 2.0 ** -6
        assert np.all(np.abs(wq[i] - w[i])[normal] <= 2.0 ** -4 * np.abs(w[i])[normal] * (1 + 1e-6))
        assert np.all(np.abs(wq[i] - w[i])[~normal] <= 2.0 ** -10 * sc[i] * (1 + 1e-6))
    w2 = w * np.float32(8.0)
    wq2, sc2 = quantize_rows(w2)
    assert np.array_equal(wq2, wq * np.float32(8.0)) and np.array_equal(sc2[sc2 != 1], (sc * 8)[sc2 != 1])


def test_fp8_weight_stack_is_the_dequantised_model():
    """With FP8 weights the oracle's step is the bf16-source model run with
    every projection replaced by its dequantised rows (checked against the
    full recompute of a model holding those rows)."""
    cfg = small_cfg(w_dtype="fp8", act_dtype="bf16", n_layers=2, d_model=512, n_heads=4, n_kv_heads=4,
                    head_dim=128, d_ffn=1024)
    model = synth.Model(cfg, gain_noise=True)
    outs, orc = _run_incremental(cfg, model, [0], 6, np.float64)

    class Dq:
        g_final = model.g_final
        kv_scale = model.kv_scale

        def layer(self, l):
            return orc.layer(l)
    full = forward_full(dict(cfg, w_dtype="bf16"), Dq(), frames(cfg, 0, 6), dtype=np.float64)
    assert rel_err(outs[0], full) < 1e-10
    plain = forward_full(dict(cfg, w_dtype="bf16"), model, frames(cfg, 0, 6), dtype=np.float64)
    assert rel_err(outs[0], plain) > 1e-3  # the quantisation is really applied
