"""The ABI checks of tests/test_abi.py against a host-sanitized build of libprism.

The library's host code (argument checks, workspace planning, dispatch) is compiled with
AddressSanitizer and UndefinedBehaviorSanitizer (host only; the device code is the same),
loaded into a child interpreter with the sanitizer runtime preloaded, and every test of
tests/test_abi.py runs against it.  Those tests call every entry point with valid and
invalid arguments but never launch a kernel, so no GPU is needed; an out-of-bounds host
access, a use after free, a signed overflow or a misaligned access in the host code aborts
the child with a report.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all",
             "-shared-libsan"]


def test_abi_under_host_sanitizers():
    rt = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rt:
        pytest.skip("no clang AddressSanitizer runtime in this ROCm installation")
    from delta_rule_sequence_amd import build as b
    obj = os.path.join(b.CSRC, "_build_asan")
    lib = os.path.join(obj, "libprism_san.so")
    b.build(extra_flags=SAN_FLAGS, lib_path=lib, obj_dir=obj)
    env = dict(os.environ, LD_PRELOAD=rt[-1], PRISM_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "tests/test_abi.py"], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, out
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out
