"""The host logic (profile validation and layout planning, the slot state
machine) built with AddressSanitizer and UndefinedBehaviorSanitizer, and
the host ABI tests run against that build in a child process: any invalid
memory access or undefined behaviour aborts the child."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    out = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return out if out and os.path.isabs(out) and os.path.exists(out) else None


def test_host_abi_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc sanitizer runtimes not installed")
    sys.path.insert(0, ROOT)
    from frame_decode_amd import build
    lib = build.build_host_sanitized(str(tmp_path / "libfd_host_san.so"))
    env = dict(os.environ)
    env.update(FD_HOST_LIB=lib, LD_PRELOAD=f"{asan}:{ubsan}",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    # the tests of the host-only library (not the two that load the HIP library)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_host_abi.py"),
                        "-k", "not exports_every_declared_symbol and not through_the_product_library"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout, tail
