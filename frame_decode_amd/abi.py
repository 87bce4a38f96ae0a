"""ctypes mirror of include/fd.h (structs, constants, prototypes)."""
from __future__ import annotations

import ctypes
import os

FD_OK = 0
FD_E_INVAL = -1
FD_E_UNSUPPORTED = -2
FD_E_NOSLOT = -3
FD_E_BADSLOT = -4
FD_E_CTXFULL = -5
FD_E_DEVICE = -6
FD_E_STATE = -7

FD_F32 = 0
FD_BF16 = 1
FD_FP8_E4M3 = 2
FD_EXEC_KERNELS, FD_EXEC_WALK = 0, 1
FD_PROJ_AUTO, FD_PROJ_F16, FD_PROJ_BF16X2 = 0, 1, 2

_DT = {"f32": FD_F32, "bf16": FD_BF16, "fp8": FD_FP8_E4M3}
PROJ_IN = {"auto": FD_PROJ_AUTO, "f16": FD_PROJ_F16, "bf16x2": FD_PROJ_BF16X2}

c_i32 = ctypes.c_int32
c_p = ctypes.c_void_p


class FdError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (status {status})")
        self.status = status


class FdConfig(ctypes.Structure):
    _fields_ = [
        ("n_layers", c_i32), ("d_model", c_i32), ("n_heads", c_i32), ("n_kv_heads", c_i32),
        ("head_dim", c_i32), ("d_ffn", c_i32), ("rms_eps", ctypes.c_float),
        ("rope_base", ctypes.c_float), ("max_slots", c_i32), ("max_context", c_i32),
        ("w_dtype", c_i32), ("act_dtype", c_i32), ("kv_dtype", c_i32),
        ("depth_steps", c_i32), ("depth_layers", c_i32), ("depth_d", c_i32),
        ("depth_heads", c_i32), ("depth_kv_heads", c_i32), ("depth_head_dim", c_i32),
        ("depth_ffn", c_i32), ("exec_mode", c_i32), ("kv_ring", c_i32), ("vocab", c_i32),
        ("proj_in", c_i32),
    ]


class FdSizes(ctypes.Structure):
    _fields_ = [("packed_weights", ctypes.c_uint64), ("kv_arena", ctypes.c_uint64),
                ("workspace", ctypes.c_uint64), ("slot_table", ctypes.c_uint64)]


class FdLayerWeights(ctypes.Structure):
    _fields_ = [(n, c_p) for n in ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down",
                                   "g_attn", "g_ffn")]


class FdWeights(ctypes.Structure):
    _fields_ = [("layers", ctypes.POINTER(FdLayerWeights)), ("g_final", c_p), ("kv_scale", c_p),
                ("w_in", c_p), ("depth_layers", ctypes.POINTER(FdLayerWeights)),
                ("depth_g_final", c_p), ("w_head", c_p)]


class FdBuffers(ctypes.Structure):
    _fields_ = [("packed_weights", c_p), ("kv_arena", c_p), ("workspace", c_p),
                ("slot_table", c_p)]


class FdKvView(ctypes.Structure):
    _fields_ = [("base", c_p), ("slot_stride", ctypes.c_uint64), ("layer_stride", ctypes.c_uint64),
                ("kv_stride", ctypes.c_uint64), ("head_stride", ctypes.c_uint64),
                ("pos_stride", ctypes.c_uint64), ("elem_bytes", c_i32), ("n_layers", c_i32),
                ("n_kv_heads", c_i32), ("max_context", c_i32), ("head_dim", c_i32),
                ("max_slots", c_i32), ("kv_scale", c_p), ("slot_active", c_p), ("slot_pos", c_p)]


EXPORTS = ["fd_plan", "fd_init", "fd_alloc_slots", "fd_step", "fd_step_tokens", "fd_step_static",
           "fd_free", "fd_destroy",
           "fd_kv_layout", "fd_set_position", "fd_slot_state", "fd_kv_write", "fd_sync",
           "fd_profile", "fd_profile_read", "fd_trace_attention", "fd_walk_abort_next", "fd_read_probe",
           "fd_last_error",
           "fd_status_str"]

FD_N_KINDS = 15
FD_STATIC_SCRATCH_BYTES = 64 << 20
KIND_NAMES = ["embed", "qkv", "attention", "o_proj", "gate_up", "down", "final", "depth_in",
              "walk", "head", "depth_qkv", "depth_attention", "depth_o_proj", "depth_gate_up",
              "depth_down"]


def config_from_dict(cfg: dict) -> FdConfig:
    c = FdConfig()
    for k in ("n_layers", "d_model", "n_heads", "n_kv_heads", "head_dim", "d_ffn",
              "max_slots", "max_context", "depth_steps", "depth_layers", "depth_d",
              "depth_heads", "depth_kv_heads", "depth_head_dim", "depth_ffn"):
        setattr(c, k, int(cfg.get(k, 0)))
    c.rms_eps = float(cfg["rms_eps"])
    c.rope_base = float(cfg["rope_base"])
    c.w_dtype = _DT[cfg["w_dtype"]]
    c.act_dtype = _DT[cfg["act_dtype"]]
    c.kv_dtype = _DT[cfg["kv_dtype"]]
    c.exec_mode = int(cfg.get("exec_mode", 0))
    c.kv_ring = int(cfg.get("kv_ring", 0))
    c.vocab = int(cfg.get("vocab", 0))
    c.proj_in = PROJ_IN[cfg.get("proj_in", "auto")]
    return c


def _proto(lib):
    P = ctypes.POINTER
    lib.fd_plan.argtypes = [P(FdConfig), P(FdSizes)]
    lib.fd_init.argtypes = [P(FdConfig), P(FdWeights), P(FdBuffers), c_p, P(c_p)]
    lib.fd_alloc_slots.argtypes = [c_p, c_i32, P(c_i32)]
    lib.fd_step.argtypes = [c_p, c_p, c_p, c_p, c_p]
    lib.fd_step_tokens.argtypes = [c_p, c_p, c_p, c_p, c_p, c_p, c_p]
    lib.fd_step_static.argtypes = [c_p, c_p, c_p, c_p, c_p]
    lib.fd_free.argtypes = [c_p, P(c_i32), c_i32]
    lib.fd_destroy.argtypes = [c_p]
    lib.fd_kv_layout.argtypes = [c_p, P(FdKvView)]
    lib.fd_set_position.argtypes = [c_p, c_i32, c_i32]
    lib.fd_slot_state.argtypes = [c_p, c_i32, P(c_i32), P(c_i32)]
    lib.fd_kv_write.argtypes = [c_p, c_i32, c_i32, c_i32, c_i32, c_p, c_p]
    lib.fd_sync.argtypes = [c_p, c_p]
    lib.fd_profile.argtypes = [c_p, c_i32]
    lib.fd_trace_attention.argtypes = [c_p, c_p, c_i32, c_i32]
    lib.fd_walk_abort_next.argtypes = [c_p]
    lib.fd_profile_read.argtypes = [c_p, P(ctypes.c_double), P(ctypes.c_int64), c_i32]
    lib.fd_read_probe.argtypes = [c_p, ctypes.c_uint64, c_p, c_i32, c_p]
    lib.fd_last_error.argtypes = [c_p]
    lib.fd_last_error.restype = ctypes.c_char_p
    lib.fd_status_str.argtypes = [c_i32]
    lib.fd_status_str.restype = ctypes.c_char_p
    for n in EXPORTS:
        if n not in ("fd_last_error", "fd_status_str"):
            getattr(lib, n).restype = c_i32


def load_library(path: str):
    if not os.path.exists(path):
        raise FdError(FD_E_STATE, f"{path} is not built (run __graft_entry__.build() or "
                                  "python -m frame_decode_amd.build)")
    lib = ctypes.CDLL(path)
    _proto(lib)
    return lib
