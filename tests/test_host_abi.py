"""Host-side logic of the C ABI, without a GPU: the built libraries load and
export every declared symbol; profile validation; buffer sizes and the
cache layout formula; the slot state machine (admission order,
all-or-nothing allocation, frees, positions, full windows)."""
import ctypes
import os
import re

import pytest

import synth
from frame_decode_amd.abi import (FD_E_BADSLOT, FD_E_INVAL, FD_E_NOSLOT, FD_E_UNSUPPORTED, FD_OK,
                                  FdConfig, FdSizes, config_from_dict)

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(ROOT, "frame_decode_amd", "libfd.so")
HOST = os.path.join(ROOT, "frame_decode_amd", "libfd_host.so")
HEADER = os.path.join(ROOT, "include", "fd.h")


def declared_symbols():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:fd_status|const char\*)\s+(fd_\w+)\s*\(", txt, re.M)))


@pytest.fixture(scope="module")
def host():
    path = os.environ.get("FD_HOST_LIB", HOST)  # (a sanitizer build of the same sources)
    if not os.path.exists(path):
        pytest.fail(f"{path} not built (run __graft_entry__.build())")
    h = ctypes.CDLL(path)
    h.fdh_pool_new.restype = ctypes.c_void_p
    h.fdh_pool_new.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
    for n in ("fdh_pool_alloc", "fdh_pool_free"):
        getattr(h, n).argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32), ctypes.c_int32]
    h.fdh_pool_alloc.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(ctypes.c_int32)]
    h.fdh_pool_set_position.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32]
    h.fdh_pool_state.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(ctypes.c_int32),
                                 ctypes.POINTER(ctypes.c_int32)]
    for n in ("fdh_pool_any_full", "fdh_pool_advance", "fdh_pool_dirty", "fdh_pool_clear_dirty",
              "fdh_pool_delete"):
        getattr(h, n).argtypes = [ctypes.c_void_p]
    h.fdh_pool_image.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32)]
    h.fdh_plan.argtypes = [ctypes.POINTER(FdConfig), ctypes.POINTER(FdSizes)]
    h.fdh_last_error.restype = ctypes.c_char_p
    h.fdh_gemm_shape.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                 ctypes.POINTER(ctypes.c_int32)]
    h.fdh_stack_shapes.argtypes = [ctypes.POINTER(FdConfig), ctypes.POINTER(ctypes.c_int32)]
    h.fdh_stack_mtiles.argtypes = [ctypes.POINTER(FdConfig), ctypes.POINTER(ctypes.c_int32)]
    h.fdh_pool_mark_stale.argtypes = [ctypes.c_void_p]
    h.fdh_pool_any_stale.argtypes = [ctypes.c_void_p]
    return h


def test_library_loads_and_exports_every_declared_symbol():
    assert os.path.exists(LIB), "libfd.so not built"
    lib = ctypes.CDLL(LIB)
    syms = declared_symbols()
    assert len(syms) >= 13
    for s in syms:
        assert hasattr(lib, s), s
    from frame_decode_amd.abi import EXPORTS
    assert sorted(EXPORTS) == syms


def test_binding_constants_match_the_header():
    """The binding's copies of the header's sizes and kernel-kind count."""
    from frame_decode_amd import abi
    text = open(os.path.join(ROOT, "include", "fd.h")).read()
    kinds = int(re.search(r"#define FD_N_KINDS (\d+)", text).group(1))
    assert abi.FD_N_KINDS == kinds == len(abi.KIND_NAMES)
    assert len(set(abi.KIND_NAMES)) == kinds


def test_fd_plan_through_the_product_library():
    """fd_plan is pure host code: callable without a GPU."""
    from frame_decode_amd import fd_plan
    s = fd_plan(synth.get_config("7b_s80_p1499"))
    # [S][L][K|V][H_kv][T][D] bytes: 80 * 32 * 2 * 32 * 1500 * 128
    assert s["kv_arena"] == 80 * 32 * 2 * 32 * 1500 * 128
    # packed weights hold at least every weight once
    assert s["packed_weights"] >= 13_153_337_344
    assert s["packed_weights"] < 13_153_337_344 * 1.01


def _plan(host, cfg):
    c = config_from_dict(cfg)
    s = FdSizes()
    st = host.fdh_plan(ctypes.byref(c), ctypes.byref(s))
    return st, s


@pytest.mark.parametrize("name", list(synth.CONFIGS))
def test_every_workload_is_supported(host, name):
    st, s = _plan(host, synth.get_config(name))
    assert st == FD_OK, host.fdh_last_error()
    cfg = synth.get_config(name)
    eb = 1 if cfg["kv_dtype"] == "fp8" else 4
    assert s.kv_arena == max(256, cfg["max_slots"] * cfg["n_layers"] * 2 * cfg["n_kv_heads"] *
                             cfg["max_context"] * cfg["head_dim"] * eb)


def test_fp8_cache_is_half_of_bf16_and_quarter_of_fp32(host):
    """The FP8 cache halves the cache bytes of a 16-bit cache (PersonaPlex
    page, "Compressing the Temporal KV cache"); fp32 is four times FP8."""
    a = synth.get_config("7b_s80_p1499")
    b = dict(a, kv_dtype="f32", w_dtype="f32", act_dtype="f32")
    _, sa = _plan(host, a)
    _, sb = _plan(host, b)
    assert sb.kv_arena == 4 * sa.kv_arena


@pytest.mark.parametrize("field,value,status", [
    ("head_dim", 96, FD_E_UNSUPPORTED),
    ("n_kv_heads", 3, FD_E_UNSUPPORTED),
    ("d_model", 100, FD_E_UNSUPPORTED),
    ("d_ffn", 0, FD_E_UNSUPPORTED),
    ("max_slots", 0, FD_E_UNSUPPORTED),
    ("max_context", 0, FD_E_UNSUPPORTED),
    ("rope_base", -1.0, FD_E_INVAL),
    ("rms_eps", float("nan"), FD_E_INVAL),
    ("act_dtype", "f32", FD_E_UNSUPPORTED),
])
def test_bad_profiles_are_rejected(host, field, value, status):
    cfg = synth.get_config("7b_s8_p256")
    cfg[field] = value
    st, _ = _plan(host, cfg)
    assert st == status
    assert host.fdh_last_error()


def test_depth_stack_needs_fp32(host):
    cfg = synth.get_config("talker_s56")
    cfg.update(w_dtype="bf16", act_dtype="bf16")
    st, _ = _plan(host, cfg)
    assert st == FD_E_UNSUPPORTED


def test_walk_mode(host):
    """The persistent walk of the whole step is planned for the three
    compiled shape families (it needs workspace for its own buffers) and
    refused for other shapes and for unknown modes."""
    for name in ("tiny", "7b_s8_p256", "7b_s80_p1499", "7b_ragged_80x56", "talker_s56"):
        cfg = synth.get_config(name)
        if cfg["act_dtype"] == "bf16":  # the walk's form of the projection inputs
            cfg["proj_in"] = "bf16x2"
        st0, s0 = _plan(host, cfg)
        cfg["exec_mode"] = 1
        st1, s1 = _plan(host, cfg)
        assert st0 == FD_OK and st1 == FD_OK and s1.workspace > s0.workspace, name
        assert s1.packed_weights == s0.packed_weights and s1.kv_arena == s0.kv_arena
        if cfg["act_dtype"] == "bf16":  # AUTO in the walk is the fp16 form
            st2, s2 = _plan(host, dict(cfg, proj_in="auto"))
            st3, s3 = _plan(host, dict(cfg, proj_in="f16"))
            assert st2 == st3 == FD_OK and (s2.packed_weights, s2.workspace) == (s3.packed_weights, s3.workspace)
            assert s3.workspace < s1.workspace  # no low parts
    # fp32 7B-shaped stack (head_dim 128 without a depth stack): not compiled
    f32 = synth.get_config("7b_s8_p256")
    f32.update(exec_mode=1, w_dtype="f32", act_dtype="f32", kv_dtype="f32")
    assert _plan(host, f32)[0] == FD_E_UNSUPPORTED
    # bf16 weights over an fp32 cache: not compiled
    bf_f32kv = synth.get_config("7b_s8_p256")
    bf_f32kv.update(exec_mode=1, kv_dtype="f32")
    assert _plan(host, bf_f32kv)[0] == FD_E_UNSUPPORTED
    # talker geometry beyond 4 row tiles per m-group
    many = synth.get_config("talker_s56")
    many.update(exec_mode=1, max_slots=80)
    assert _plan(host, many)[0] == FD_E_UNSUPPORTED
    bad = synth.get_config("talker_s56")
    bad["exec_mode"] = 7
    assert _plan(host, bad)[0] == FD_E_INVAL


def test_projection_input_forms(host):
    """bf16 profiles: AUTO is the fp16 form in either mode; the fp16 form
    stores one fp32 scale per output row after each matrix's tiles and needs
    no low-part buffers; fp32 profiles take only AUTO; unknown values are
    refused."""
    from frame_decode_amd import abi
    text = open(os.path.join(ROOT, "include", "fd.h")).read()
    for n in ("FD_PROJ_AUTO", "FD_PROJ_F16", "FD_PROJ_BF16X2"):
        assert int(re.search(rf"#define {n}\s+(\d+)", text).group(1)) == getattr(abi, n)
    cfg = synth.get_config("7b_s80_p1499")
    (st_a, a), (st_f, f), (st_b, b) = (_plan(host, dict(cfg, proj_in=v)) for v in ("auto", "f16", "bf16x2"))
    assert st_a == st_f == st_b == FD_OK
    assert (a.packed_weights, a.workspace) == (f.packed_weights, f.workspace)
    rows = 32 * (12288 + 4096 + 22528 + 4096)  # output rows of every projection
    assert f.packed_weights - b.packed_weights == 4 * rows
    # low parts of xg, h and o: 80 rows x (4096 + 11264 + 4096) x 2 bytes (an
    # unused region still takes its 256-byte alignment unit)
    assert b.workspace - f.workspace == 80 * (4096 + 11264 + 4096) * 2 - 3 * 256
    assert _plan(host, dict(cfg, proj_in="f16", exec_mode=1))[0] == FD_OK
    assert _plan(host, dict(cfg, proj_in="bf16x2", exec_mode=1))[0] == FD_OK
    fp8 = dict(cfg, w_dtype="fp8")
    assert _plan(host, dict(fp8, proj_in="f16"))[0] == FD_OK
    assert _plan(host, dict(fp8, proj_in="bf16x2"))[0] == FD_OK
    tiny = synth.get_config("tiny")
    assert _plan(host, dict(tiny, proj_in="auto"))[0] == FD_OK
    for v in ("f16", "bf16x2"):
        assert _plan(host, dict(tiny, proj_in=v))[0] == FD_E_UNSUPPORTED
    c = config_from_dict(cfg)
    c.proj_in = 3
    assert host.fdh_plan(ctypes.byref(c), ctypes.byref(FdSizes())) == FD_E_UNSUPPORTED


def test_gemm_tiling_covers_the_projection(host):
    out = (ctypes.c_int32 * 9)()
    for (N, K, wt, MT) in [(12288, 4096, 1, 5), (4096, 11264, 1, 5), (22528, 4096, 1, 1),
                           (1536, 1152, 0, 4), (1024, 2816, 0, 4), (4096, 4096, 1, 47)]:
        host.fdh_gemm_shape(N, K, wt, MT, out)
        NB, KB, R, P, MG, MTG, ng, grid, KT = list(out)
        assert NB * 16 == N and KB * KT == K
        assert ng * R >= NB and R in (4, 6) and MG * MTG >= MT and MTG <= 8
        assert 1 <= P <= KB and grid == ng * P * MG


def _stack_shapes(host, cfg):
    out = (ctypes.c_int32 * 32)()
    st = host.fdh_stack_shapes(ctypes.byref(config_from_dict(cfg)), out)
    assert st == FD_OK, host.fdh_last_error()
    v = list(out)
    names = ("qkv", "o", "gu", "down", "d.qkv", "d.o", "d.gu", "d.down")
    return {n: tuple(v[4 * i:4 * i + 4]) for i, n in enumerate(names) if v[4 * i]}


def test_row_split_projection_plan(host, monkeypatch):
    """By default every projection takes the k-split variant (4 or 6 blocks
    per workgroup); a tuning override selects the row-split variant (bf16
    weights in the kernel sequence, two-part or fp16 rows: not the
    persistent walk, FP8 weights or fp32 stacks), with two k-halves only
    where each split's k-tiles divide evenly."""
    monkeypatch.delenv("FD_TUNE", raising=False)
    cfg = synth.get_config("7b_s80_p1499")
    cfg["proj_in"] = "bf16x2"  # (the variant takes the rows as two bf16 parts)
    sh = _stack_shapes(host, cfg)
    assert all(sh[n][0] in (4, 6) and sh[n][2] == 1 for n in sh)
    assert sh["gu"] == (6, 1, 1, 235)  # 1408 blocks in groups of 6, no k-split
    row_split = "gu.NG=12,gu.P=2,gu.KH=2"
    monkeypatch.setenv("FD_TUNE", row_split)
    assert _stack_shapes(host, cfg)["gu"] == (12, 2, 2, 236)  # 118 n-groups x 2 k-splits
    assert _stack_shapes(host, dict(cfg, proj_in="f16"))["gu"] == (12, 2, 2, 236)  # fp16 rows too
    assert _stack_shapes(host, dict(cfg, exec_mode=1))["gu"][0] in (4, 6)
    assert _stack_shapes(host, dict(cfg, w_dtype="fp8"))["gu"][0] in (4, 6)
    assert _stack_shapes(host, dict(synth.get_config("talker_s56"), exec_mode=0))["gu"][0] in (4, 6)
    monkeypatch.setenv("FD_TUNE", "qkv.NG=12,qkv.P=4,qkv.KH=2,o.NG=8,o.P=8,down.NG=16,down.P=11,down.KH=2")
    sh = _stack_shapes(host, cfg)
    assert sh["qkv"] == (12, 4, 2, 256)
    assert sh["o"] == (8, 8, 1, 256)
    assert sh["down"] == (16, 11, 2, 176)  # 352 k-tiles / 11 splits = 32 per split
    monkeypatch.setenv("FD_TUNE", "down.NG=12,down.P=32,down.KH=2,o.NG=12,o.P=32,o.KH=2")
    sh = _stack_shapes(host, cfg)
    assert sh["down"] == (12, 32, 1, 704)  # 11 k-tiles per split: no even halves
    assert sh["o"] == (12, 32, 2, 704)  # 4 k-tiles per split: two steps of two


def test_one_block_projections_for_fp32_stacks(host, monkeypatch):
    """fp32 stacks in the kernel sequence cut the k-split to none or 2 with
    two or one weight blocks per workgroup where that still fills two
    thirds of the CUs (the talker's depth gate/up with two blocks and its
    depth QKV with one, no split; its main QKV with 2 splits of one), and
    take two blocks where those fill as many CUs as four with fewer splits
    (its O and down projections); the main gate/up, where two blocks only
    tie, keeps four.  With the opt-in three-product loop (tiles of 32 k, no
    6-block shapes) the depth QKV takes 2 splits of two blocks.  The
    persistent walk and bf16 stacks keep 4 or 6 blocks per workgroup."""
    monkeypatch.delenv("FD_TUNE", raising=False)
    talker = dict(synth.get_config("talker_s56"), exec_mode=0)
    sh = _stack_shapes(host, talker)
    assert sh["qkv"] == (1, 2, 1, 192)      # 96 blocks x 2 splits (9 splits of 4 blocks before)
    assert sh["d.qkv"] == (1, 1, 1, 192)    # 192 blocks, no split (8 splits of 6 before)
    assert sh["d.gu"] == (2, 1, 1, 176)     # 176 pairs of blocks, no split, no reduce launch
    assert sh["o"] == (2, 4, 1, 144)        # 36 pairs of blocks x 4 splits
    assert sh["down"] == (2, 6, 1, 216)     # 432 k-tiles in 6 splits (12 of 4 blocks before)
    assert sh["d.o"] == (2, 8, 1, 256) and sh["d.down"] == (2, 8, 1, 256)  # 16 splits before
    assert sh["gu"] == (4, 1, 1, 216)
    walk = _stack_shapes(host, dict(talker, exec_mode=1))
    assert all(v[0] in (4, 6) for v in walk.values())
    big = _stack_shapes(host, synth.get_config("7b_s80_p1499"))
    assert set(big) == {"qkv", "o", "gu", "down"} and all(v[0] in (4, 6) for v in big.values())
    monkeypatch.setenv("FD_TUNE", "d.gu.NG=6,d.gu.P=4,o.NG=1,o.P=2")
    sh = _stack_shapes(host, talker)
    assert sh["d.gu"] == (6, 4, 1, 236) and sh["o"] == (1, 2, 1, 144)
    monkeypatch.setenv("FD_TUNE", "x3=1")
    sh = _stack_shapes(host, talker)
    assert sh["d.qkv"] == (2, 2, 1, 192)    # 96 pairs of blocks x 2 splits
    monkeypatch.setenv("FD_TUNE", "x3=1,qkv.NG=6,d.gu.NG=4,d.gu.P=4")
    sh = _stack_shapes(host, talker)
    assert sh["qkv"][0] == 1  # (6 blocks: not built for the three-product loop)
    assert sh["d.gu"] == (4, 4, 1, 352)     # 32 k-tiles of 32 in 4 splits
    assert _stack_shapes(host, dict(talker, exec_mode=1))["o"][0] in (4, 6)


class Pool:
    def __init__(self, h, n, T, rolling=0):
        self.h = h
        self.p = h.fdh_pool_new(n, T, rolling)
        self.n = n

    def alloc(self, k):
        out = (ctypes.c_int32 * max(1, k))()
        st = self.h.fdh_pool_alloc(self.p, k, out)
        return st, [out[i] for i in range(k)]

    def free(self, ids):
        arr = (ctypes.c_int32 * max(1, len(ids)))(*ids)
        return self.h.fdh_pool_free(self.p, arr, len(ids))

    def state(self, s):
        a, p = ctypes.c_int32(), ctypes.c_int32()
        st = self.h.fdh_pool_state(self.p, s, ctypes.byref(a), ctypes.byref(p))
        return st, a.value, p.value

    def image(self):
        """active[S] + pos[S] (the attention order is checked separately)."""
        return self.full_image()[:2 * self.n]

    def full_image(self):
        out = (ctypes.c_int32 * (3 * self.n))()
        self.h.fdh_pool_image(self.p, out)
        return list(out)


def test_attention_order_is_longest_first(host):
    """The slot table's third part orders the slots for attention: active
    slots by descending position (ties by slot number), then the inactive
    slots ascending; a permutation of every slot, refreshed with the table."""
    P = Pool(host, 7, 100)
    st, ids = P.alloc(5)
    assert st == FD_OK and ids == [0, 1, 2, 3, 4]
    for s, p in zip(ids, [10, 70, 10, 99, 0]):
        assert host.fdh_pool_set_position(P.p, s, p) == FD_OK
    assert P.free([2]) == FD_OK
    img = P.full_image()
    order = img[14:]
    assert order == [3, 1, 0, 4, 2, 5, 6]
    assert sorted(order) == list(range(7))
    act, pos = img[:7], img[7:14]
    lens = [pos[s] for s in order if act[s]]
    assert lens == sorted(lens, reverse=True)


def test_slot_state_machine(host):
    P = Pool(host, 5, 10)
    st, ids = P.alloc(3)
    assert st == FD_OK and ids == [0, 1, 2]
    assert P.free([1]) == FD_OK
    st, ids = P.alloc(2)
    assert st == FD_OK and ids == [1, 3]  # lowest free first
    before = P.image()
    st, _ = P.alloc(2)  # only slot 4 is free: all or nothing
    assert st == FD_E_NOSLOT and P.image() == before
    # double free / unallocated / out of range / repeated: rejected, no change
    assert P.free([4]) == FD_E_BADSLOT
    assert P.free([0, 0]) == FD_E_BADSLOT
    assert P.free([0, 7]) == FD_E_BADSLOT
    assert P.free([-1]) == FD_E_BADSLOT
    assert P.image() == before
    assert P.free([0, 3]) == FD_OK
    assert P.state(0)[1] == 0 and P.state(3)[1] == 0


def test_positions_advance_and_full_window(host):
    P = Pool(host, 3, 4)
    _, ids = P.alloc(2)
    assert host.fdh_pool_set_position(P.p, 0, 3) == FD_OK
    assert host.fdh_pool_set_position(P.p, 2, 1) == FD_E_BADSLOT  # not allocated
    assert host.fdh_pool_set_position(P.p, 1, 5) == FD_E_INVAL    # beyond the window
    assert host.fdh_pool_any_full(P.p) == -1
    host.fdh_pool_advance(P.p)
    assert P.state(0)[1:] == (1, 4) and P.state(1)[1:] == (1, 1)
    assert P.state(2)[1:] == (0, 0)  # inactive slots do not advance
    assert host.fdh_pool_any_full(P.p) == 0
    # re-admission starts at position 0
    assert P.free([0]) == FD_OK
    st, ids = P.alloc(1)
    assert ids == [0] and P.state(0)[1:] == (1, 0)


def test_rolling_window_positions(host):
    """With a rolling window a session keeps stepping past the window
    length; only the largest frame index (2^30) stops it."""
    P = Pool(host, 2, 4, rolling=1)
    P.alloc(1)
    assert host.fdh_pool_set_position(P.p, 0, 3) == FD_OK
    host.fdh_pool_advance(P.p)
    host.fdh_pool_advance(P.p)
    assert P.state(0)[1:] == (1, 5) and host.fdh_pool_any_full(P.p) == -1
    assert host.fdh_pool_set_position(P.p, 0, 1000) == FD_OK
    assert host.fdh_pool_set_position(P.p, 0, (1 << 30) + 1) == FD_E_INVAL
    assert host.fdh_pool_set_position(P.p, 0, 1 << 30) == FD_OK
    assert host.fdh_pool_any_full(P.p) == 0


def test_rolling_window_plan(host):
    """kv_ring 0 and 1 plan with the same buffer sizes; other values are
    invalid arguments."""
    cfg = synth.get_config("7b_s8_p256")
    st0, s0 = _plan(host, cfg)
    cfg["kv_ring"] = 1
    st1, s1 = _plan(host, cfg)
    assert st0 == FD_OK and st1 == FD_OK
    assert (s0.packed_weights, s0.kv_arena, s0.workspace) == (s1.packed_weights, s1.kv_arena, s1.workspace)
    cfg["kv_ring"] = 2
    assert _plan(host, cfg)[0] == FD_E_INVAL


def test_device_image_layout(host):
    P = Pool(host, 4, 8)
    P.alloc(2)
    host.fdh_pool_set_position(P.p, 1, 5)
    assert P.image() == [1, 1, 0, 0, 0, 5, 0, 0]
    host.fdh_pool_clear_dirty(P.p)
    assert host.fdh_pool_dirty(P.p) == 0
    host.fdh_pool_set_position(P.p, 0, 2)
    assert host.fdh_pool_dirty(P.p) == 1


def test_output_head_plan(host):
    """A vocabulary adds exactly the head's tiles to the packed weights (and,
    as fp16 codes, one fp32 scale per row); sizes that are not a multiple of
    16 are refused."""
    cfg = synth.get_config("7b_s8_p256")
    st0, s0 = _plan(host, cfg)
    cfg["vocab"] = 2048
    st1, s1 = _plan(host, cfg)
    assert st0 == FD_OK and st1 == FD_OK
    assert s1.packed_weights - s0.packed_weights == 2048 * 4096 * 2 + 2048 * 4
    st2, s2 = _plan(host, dict(cfg, proj_in="bf16x2"))
    st3, s3 = _plan(host, dict(cfg, proj_in="bf16x2", vocab=0))
    assert st2 == st3 == FD_OK and s2.packed_weights - s3.packed_weights == 2048 * 4096 * 2
    assert s1.kv_arena == s0.kv_arena and s1.workspace > s0.workspace
    cfg["vocab"] = 2050
    assert _plan(host, cfg)[0] == FD_E_UNSUPPORTED


def test_fp8_weight_plan(host):
    """FP8 weights: one byte per parameter plus one fp32 scale per output
    row; bf16 activations required; no depth stack and no persistent walk."""
    cfg = synth.get_config("7b_s8_p256")
    cfg["proj_in"] = "bf16x2"  # (bf16 weights as they are)
    st0, s0 = _plan(host, cfg)
    cfg.update(w_dtype="fp8", act_dtype="bf16")
    st1, s1 = _plan(host, cfg)
    assert st0 == FD_OK and st1 == FD_OK
    params = 32 * (12288 * 4096 + 4096 * 4096 + 22528 * 4096 + 4096 * 11264)
    rows = 32 * (12288 + 4096 + 22528 + 4096)
    # weights halve; tables (gains, rope, scales of the cache) are common to both
    assert s0.packed_weights - s1.packed_weights == params - 4 * rows
    assert s1.kv_arena == s0.kv_arena
    bad = dict(cfg, act_dtype="fp8")
    assert _plan(host, bad)[0] == FD_E_UNSUPPORTED
    walk = dict(cfg, exec_mode=1)
    assert _plan(host, walk)[0] == FD_E_UNSUPPORTED
    talker = synth.get_config("talker_s56")
    talker.update(w_dtype="fp8", act_dtype="bf16")
    assert _plan(host, talker)[0] == FD_E_UNSUPPORTED


@pytest.mark.parametrize("slots", [7, 80, 96, 112, 128, 140, 709, 4096])
def test_fp8_weight_row_groups_stay_within_the_built_kernels(host, slots):
    """FP8-weight projections are built for at most 5 row tiles per m-group:
    every slot count plans within that (rows padded to whole m-groups), and
    bf16 profiles keep their own limit of 8."""
    for wdt, cap in (("fp8", 5), ("bf16", 8)):
        cfg = synth.scaled_config("7b_s80_p1499", max_slots=slots, w_dtype=wdt, act_dtype="bf16",
                                  vocab=1024)
        for k in ("position",):
            cfg.pop(k, None)
        out = (ctypes.c_int32 * 11)()
        assert host.fdh_stack_mtiles(ctypes.byref(config_from_dict(cfg)), out) == FD_OK
        mt = out[0]
        assert mt * 16 >= slots and (mt - 1) * 16 < slots + 16 * cap
        for i in range(5):
            mg, mtg = out[1 + 2 * i], out[2 + 2 * i]
            assert 1 <= mtg <= cap, (wdt, slots, i, mtg)
            assert mg * mtg == mt, (wdt, slots, i, mg, mtg, mt)


@pytest.mark.parametrize("slots", [1, 7, 16, 33, 56, 80, 81, 96, 128, 140, 200, 709])
def test_fp32_block_counts_stay_within_the_built_kernels(host, slots, monkeypatch):
    """One- and two-block projections are built for fp32 weights with at
    most 5 row tiles per m-group: at every slot count the fp32 plan (main
    and depth stack) picks them only there, and the persistent walk (where
    it takes the profile) keeps 4 or 6 blocks."""
    monkeypatch.delenv("FD_TUNE", raising=False)
    base = synth.scaled_config("talker_s56", max_slots=slots)
    base.pop("position", None)
    for mode in (0, 1):
        cfg = dict(base, exec_mode=mode)
        mt_out = (ctypes.c_int32 * 11)()
        st = host.fdh_stack_mtiles(ctypes.byref(config_from_dict(cfg)), mt_out)
        if mode == 1 and st == FD_E_UNSUPPORTED:
            continue  # (the walk is built for a few row tilings only)
        assert st == FD_OK, host.fdh_last_error()
        mtg = {n: mt_out[2 + 2 * i] for i, n in enumerate(("qkv", "o", "gu", "down"))}
        sh = _stack_shapes(host, cfg)
        assert set(sh) == {"qkv", "o", "gu", "down", "d.qkv", "d.o", "d.gu", "d.down"}
        for n, (R, P, kh, grid) in sh.items():
            assert R in ((1, 2, 4, 6) if mode == 0 else (4, 6)), (slots, mode, n, R)
            if R in (1, 2, 6):
                # (the depth stack has the main stack's rows, so the same tiling)
                assert mtg[n.split(".")[-1]] <= 5, (slots, n, R)
            assert P >= 1 and kh == 1 and grid % P == 0
    # the opt-in three-product loop is built for 1, 2 and 4 blocks and at
    # most 5 row tiles per m-group (the rows are padded to such m-groups)
    monkeypatch.setenv("FD_TUNE", "x3=1")
    cfg = dict(base, exec_mode=0)
    mt_out = (ctypes.c_int32 * 11)()
    assert host.fdh_stack_mtiles(ctypes.byref(config_from_dict(cfg)), mt_out) == FD_OK
    assert all(1 <= mt_out[2 + 2 * i] <= 5 for i in range(4))
    assert mt_out[1] * mt_out[2] == mt_out[0] and mt_out[0] * 16 >= slots
    assert all(v[0] in (1, 2, 4) for v in _stack_shapes(host, cfg).values())


def test_stale_slots_after_an_interrupted_step(host):
    """A step that stopped early marks every active slot stale; each slot
    leaves that state when given a position or freed, and a newly admitted
    slot is never stale."""
    p = host.fdh_pool_new(4, 100, 0)
    try:
        out = (ctypes.c_int32 * 4)()
        assert host.fdh_pool_alloc(p, 3, out) == FD_OK
        assert host.fdh_pool_any_stale(p) == -1
        host.fdh_pool_mark_stale(p)
        assert host.fdh_pool_any_stale(p) == 0
        assert host.fdh_pool_set_position(p, 0, 5) == FD_OK
        assert host.fdh_pool_any_stale(p) == 1
        ids = (ctypes.c_int32 * 1)(1)
        assert host.fdh_pool_free(p, ids, 1) == FD_OK
        assert host.fdh_pool_any_stale(p) == 2
        assert host.fdh_pool_set_position(p, 2, 0) == FD_OK
        assert host.fdh_pool_any_stale(p) == -1
        one = (ctypes.c_int32 * 1)()
        assert host.fdh_pool_alloc(p, 1, one) == FD_OK and one[0] == 1
        assert host.fdh_pool_any_stale(p) == -1
    finally:
        host.fdh_pool_delete(p)
