"""The library's host code (plans, argument checks, launch set-up in
moe_api.cpp) under AddressSanitizer and UndefinedBehaviorSanitizer: the ABI
tests run against libmoe_hostsan.so with the sanitizer runtime preloaded, in
a process of their own, and any report fails them (no GPU)."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        return None
    r = subprocess.run([hipcc, "--print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def test_abi_tests_pass_with_host_sanitizers():
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("hipcc's AddressSanitizer runtime not found")
    sys.path.insert(0, ROOT)
    from routing_capacity_dispatch_amd import build
    lib = build.build_hostsan()
    env = dict(os.environ, MOE_LIB=lib, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-q", "-x",
                        "-m", "not gpu", "-p", "no:cacheprovider"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-3000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-3000:]
    assert " passed" in out
