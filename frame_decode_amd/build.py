"""Builds the HIP library (libfd.so, gfx950) and the host-only test library
(libfd_host.so) in-tree, next to this file.

    python -m frame_decode_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)

LIB = os.path.join(HERE, "libfd.so")
HOST_LIB = os.path.join(HERE, "libfd_host.so")

HIP_SOURCES = ["kernels.hip", "fd_static.hip", "fd_api.cpp", "fd_plan.cpp"]
HOST_SOURCES = ["host_shim.cpp", "fd_plan.cpp"]

# Packed fp32 VALU instructions are disabled for the device code (the
# compiler would otherwise form them from plain fp32 code); the host pass
# prints a harmless "not a recognized feature" warning for it.
# MFMA accumulators in ordinary VGPRs (amdgpu-mfma-vgpr-form): with the
# default AGPR form the projection loops copied accumulators between the
# two register files every iteration (about 1.5 move instructions per MFMA
# at six blocks per workgroup) and spilled at five row tiles in the walk.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


def _run(cmd):
    r = subprocess.run(cmd, cwd=CSRC, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{err}\n{r.stdout}")
    if err.strip():
        print(err, file=sys.stderr)


def build_host() -> str:
    tmp = HOST_LIB + ".tmp"
    _run(["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-Wall", *HOST_SOURCES, "-o", tmp])
    os.replace(tmp, HOST_LIB)
    return HOST_LIB


def build_host_sanitized(out: str) -> str:
    """The host-only library with AddressSanitizer and UndefinedBehavior-
    Sanitizer (host compiler only; no device code is involved), for running
    the host ABI tests under the sanitizers."""
    _run(["g++", "-O1", "-g", "-std=c++17", "-fPIC", "-shared", "-Wall", "-fno-omit-frame-pointer",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", *HOST_SOURCES, "-o", out])
    return out


def build_hip() -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB + ".tmp"
    _run([hipcc, *HIPCC_FLAGS, *HIP_SOURCES, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


def build_all() -> None:
    build_host()
    build_hip()


if __name__ == "__main__":
    build_all()
    print("built", LIB, HOST_LIB)
