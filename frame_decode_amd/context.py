"""Context: one serving profile on one GPU, driven through the C ABI.

Method names follow the C calls (fd_alloc_slots, fd_step, ...).  Buffers
are torch uint8 device tensors sized by fd_plan; the weights passed in are
torch device tensors in nn.Linear [out, in] layout (bf16 or fp32), gains
and FP8 scales fp32.
"""
from __future__ import annotations

import ctypes

import torch

from . import abi
from .abi import (FdBuffers, FdConfig, FdError, FdKvView, FdLayerWeights, FdSizes, FdWeights,
                  config_from_dict)


def _lib():
    from . import lib
    return lib()


def _check(st: int, ctx=None):
    if st != abi.FD_OK:
        L = _lib()
        msg = L.fd_last_error(ctx).decode() if ctx is not None else L.fd_last_error(None).decode()
        raise FdError(st, f"{L.fd_status_str(st).decode()}: {msg}")


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


def fd_plan(cfg: dict) -> dict:
    c = config_from_dict(cfg)
    s = FdSizes()
    _check(_lib().fd_plan(ctypes.byref(c), ctypes.byref(s)))
    return {"packed_weights": s.packed_weights, "kv_arena": s.kv_arena,
            "workspace": s.workspace, "slot_table": s.slot_table}


def fd_read_probe(buf, sink, grid: int, stream=None) -> None:
    """Enqueue one streaming read of the whole uint8 device tensor ``buf``."""
    _check(_lib().fd_read_probe(ctypes.c_void_p(_ptr(buf)), int(buf.numel() * buf.element_size()),
                                ctypes.c_void_p(_ptr(sink)), int(grid),
                                ctypes.c_void_p(_stream_handle(stream))))


def _stream_handle(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


class Context:
    """Owns the device buffers and the fd_ctx of one profile.

    weights: {"layers": [ {wq, wk, wv, wo, w_gate, w_up, w_down, g_attn,
    g_ffn} ...], "g_final", "kv_scale" (FP8 caches), with a depth stack
    "w_in", "depth_layers", "depth_g_final", and with a vocabulary "w_head"}
    as torch device tensors.
    """

    def __init__(self, cfg: dict, weights: dict, device="cuda", stream=None):
        self.cfg = dict(cfg)
        self.device = torch.device(device)
        self._c = config_from_dict(cfg)
        self.sizes = fd_plan(cfg)
        mk = lambda n: torch.empty(max(int(n), 256), dtype=torch.uint8, device=self.device)  # noqa: E731
        self.packed = mk(self.sizes["packed_weights"])
        self.arena = mk(self.sizes["kv_arena"])
        self.workspace = mk(self.sizes["workspace"])
        self.slot_table = mk(self.sizes["slot_table"])
        self._keep = []  # ctypes arrays referenced by FdWeights during init

        def layer_array(layers):
            arr = (FdLayerWeights * max(1, len(layers)))()
            for i, lw in enumerate(layers):
                for n in ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down", "g_attn", "g_ffn"):
                    setattr(arr[i], n, _ptr(lw[n]))
            self._keep.append(arr)
            return arr

        w = FdWeights()
        w.layers = layer_array(weights["layers"])
        w.g_final = _ptr(weights["g_final"])
        w.kv_scale = _ptr(weights.get("kv_scale"))
        if cfg.get("depth_steps", 0):
            w.w_in = _ptr(weights["w_in"])
            w.depth_layers = layer_array(weights["depth_layers"])
            w.depth_g_final = _ptr(weights["depth_g_final"])
        if cfg.get("vocab", 0):
            w.w_head = _ptr(weights["w_head"])
        b = FdBuffers(_ptr(self.packed), _ptr(self.arena), _ptr(self.workspace),
                      _ptr(self.slot_table))
        self._ctx = ctypes.c_void_p()
        _check(_lib().fd_init(ctypes.byref(self._c), ctypes.byref(w), ctypes.byref(b),
                              ctypes.c_void_p(_stream_handle(stream)), ctypes.byref(self._ctx)))
        self._keep.clear()

    # -- C calls ------------------------------------------------------------
    def fd_alloc_slots(self, n: int) -> list[int]:
        out = (ctypes.c_int32 * max(1, n))()
        _check(_lib().fd_alloc_slots(self._ctx, n, out), self._ctx)
        return [int(out[i]) for i in range(n)]

    def fd_free(self, slots) -> None:
        arr = (ctypes.c_int32 * max(1, len(slots)))(*[int(s) for s in slots])
        _check(_lib().fd_free(self._ctx, arr, len(slots)), self._ctx)

    def fd_step(self, x_in, y_out, depth_out=None, stream=None) -> None:
        _check(_lib().fd_step(self._ctx, ctypes.c_void_p(_ptr(x_in)), ctypes.c_void_p(_ptr(y_out)),
                              ctypes.c_void_p(_ptr(depth_out)),
                              ctypes.c_void_p(_stream_handle(stream))), self._ctx)

    def fd_step_static(self, x_in, y_out, depth_out=None, stream=None) -> None:
        """fd_step with the library's static device scratch as the workspace
        (allocates nothing; calls on one GPU must not overlap)."""
        _check(_lib().fd_step_static(self._ctx, ctypes.c_void_p(_ptr(x_in)), ctypes.c_void_p(_ptr(y_out)),
                                     ctypes.c_void_p(_ptr(depth_out)),
                                     ctypes.c_void_p(_stream_handle(stream))), self._ctx)

    def fd_step_tokens(self, x_in, y_out, tokens_out, logits_out=None, depth_out=None, stream=None) -> None:
        """fd_step plus the output head: tokens_out int32 [max_slots], optional
        logits_out fp32 [max_slots][vocab] (device tensors)."""
        _check(_lib().fd_step_tokens(self._ctx, ctypes.c_void_p(_ptr(x_in)), ctypes.c_void_p(_ptr(y_out)),
                                     ctypes.c_void_p(_ptr(depth_out)), ctypes.c_void_p(_ptr(tokens_out)),
                                     ctypes.c_void_p(_ptr(logits_out)),
                                     ctypes.c_void_p(_stream_handle(stream))), self._ctx)

    def fd_set_position(self, slot: int, pos: int) -> None:
        _check(_lib().fd_set_position(self._ctx, slot, pos), self._ctx)

    def fd_slot_state(self, slot: int) -> tuple[int, int]:
        a, p = ctypes.c_int32(), ctypes.c_int32()
        _check(_lib().fd_slot_state(self._ctx, slot, ctypes.byref(a), ctypes.byref(p)), self._ctx)
        return int(a.value), int(p.value)

    def fd_kv_write(self, slot: int, layer: int, t0: int, values: torch.Tensor, stream=None) -> None:
        """values: fp32 device tensor [2][n_kv_heads][n][head_dim]."""
        assert values.dtype == torch.float32 and values.is_contiguous() and values.dim() == 4
        _check(_lib().fd_kv_write(self._ctx, slot, layer, t0, int(values.shape[2]),
                                  ctypes.c_void_p(_ptr(values)),
                                  ctypes.c_void_p(_stream_handle(stream))), self._ctx)

    def fd_kv_layout(self) -> dict:
        v = FdKvView()
        _check(_lib().fd_kv_layout(self._ctx, ctypes.byref(v)), self._ctx)
        return {f: getattr(v, f) for f, _ in FdKvView._fields_}

    def fd_trace_attention(self, stamps=None, layer: int = 0) -> None:
        """Device-clock stamps of one layer's attention launch into the int64
        device tensor ``stamps`` [workgroups][4] (None turns it off)."""
        n = 0 if stamps is None else stamps.numel() // 4
        _check(_lib().fd_trace_attention(self._ctx, ctypes.c_void_p(_ptr(stamps)), int(layer), int(n)),
               self._ctx)

    def fd_walk_abort_next(self) -> None:
        """The next step's persistent walk starts with its abort flag set
        (every workgroup leaves at its first barrier wait)."""
        _check(_lib().fd_walk_abort_next(self._ctx), self._ctx)

    def fd_profile(self, enable: bool) -> None:
        _check(_lib().fd_profile(self._ctx, 1 if enable else 0), self._ctx)

    def fd_profile_read(self) -> dict:
        """{kind: (total ms, launches)} since the last read."""
        n = abi.FD_N_KINDS
        ms = (ctypes.c_double * n)()
        cnt = (ctypes.c_int64 * n)()
        _check(_lib().fd_profile_read(self._ctx, ms, cnt, n), self._ctx)
        return {abi.KIND_NAMES[k]: (float(ms[k]), int(cnt[k])) for k in range(n)}

    def fd_sync(self, stream=None) -> None:
        _check(_lib().fd_sync(self._ctx, ctypes.c_void_p(_stream_handle(stream))), self._ctx)

    def fd_destroy(self) -> None:
        if self._ctx:
            _check(_lib().fd_destroy(self._ctx))
            self._ctx = ctypes.c_void_p()

    def __del__(self):
        try:
            self.fd_destroy()
        except Exception:
            pass

    # -- views --------------------------------------------------------------
    def arena_view(self) -> torch.Tensor:
        """The cache arena as a [S][L][2][H_kv][T][D] tensor (uint8 codes or fp32)."""
        c = self.cfg
        eb = 1 if c["kv_dtype"] == "fp8" else 4
        n = c["max_slots"] * c["n_layers"] * 2 * c["n_kv_heads"] * c["max_context"] * c["head_dim"]
        t = self.arena[: n * eb]
        if eb == 4:
            t = t.view(torch.float32)
        return t.view(c["max_slots"], c["n_layers"], 2, c["n_kv_heads"], c["max_context"],
                      c["head_dim"])

    def slot_table_view(self) -> torch.Tensor:
        """Device slot table as int32 [3][S]: active flags, positions, and
        the order attention takes the slots in."""
        S = self.cfg["max_slots"]
        return self.slot_table[: 12 * S].view(torch.int32).view(3, S)
