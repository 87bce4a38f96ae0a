"""Python binding of the frame-synchronous decode step library (libfd.so).

Argument marshalling only: every step of the decode path runs in the HIP
kernels behind the C ABI declared in include/fd.h.  torch is used for device
memory (uint8 tensors sized by fd_plan) and streams.  If the built library
is missing, importing this package raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

from .abi import (FD_OK, FD_E_INVAL, FD_E_UNSUPPORTED, FD_E_NOSLOT, FD_E_BADSLOT,  # noqa: F401
                  FD_E_CTXFULL, FD_E_DEVICE, FD_E_STATE, FD_F32, FD_BF16, FD_FP8_E4M3,
                  FD_EXEC_KERNELS, FD_EXEC_WALK,
                  FdConfig, FdSizes, FdKvView, FdError, config_from_dict, load_library)

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfd.so")

_lib = None


def lib():
    """The loaded libfd.so (raises FdError if it has not been built)."""
    global _lib
    if _lib is None:
        _lib = load_library(LIB_PATH)
    return _lib


from .context import Context, fd_plan, fd_read_probe  # noqa: E402,F401
