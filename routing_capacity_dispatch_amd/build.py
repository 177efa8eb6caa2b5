"""Build libmoe.so (the C-ABI library) for gfx950 with hipcc, in-tree.

    python -m routing_capacity_dispatch_amd.build [-v]
    python -m routing_capacity_dispatch_amd.build --host-sanitize [-v]

Always recompiles.  Sources: csrc/*.hip and csrc/moe_api.cpp; the public
header is include/moe.h at the repository root.

--host-sanitize builds libmoe_hostsan.so beside libmoe.so: the host code of
moe_api.cpp (plans, argument checks, launch set-up) under AddressSanitizer
and UndefinedBehaviorSanitizer, the device code unchanged.  Load it with the
sanitizer runtime preloaded, e.g.

    LD_PRELOAD=$(hipcc --print-file-name=libclang_rt.asan-x86_64.so) \
    MOE_LIB=.../libmoe_hostsan.so python -m pytest tests/test_abi.py -m "not gpu"
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmoe.so")
LIB_HOSTSAN = os.path.join(PKG, "libmoe_hostsan.so")
BUILD_DIR = os.path.join(PKG, "_build")
ARCH = os.environ.get("MOE_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    f"--offload-arch={ARCH}",
    # gfx950: keep the compiler from emitting packed fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-parameter",
    # gemm_core.h sets M0 in inline assembly for its global -> LDS loads
    "-Wno-inline-asm",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


# host-side sanitizers only (each -fsanitize= right after -Xarch_host: the
# device code is not instrumented)
HOST_SAN = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=all",
            "-Xarch_host", "-shared-libsan", "-g"]


def _compile(src: str, verbose: bool, extra=(), suffix: str = ".o") -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + suffix)
    cmd = [hipcc(), *COMMON, *extra, "-x", "hip", "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    if verbose and out.strip():
        print(out, flush=True)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + [os.path.join(CSRC, "moe_api.cpp")]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


def build_hostsan(verbose: bool = False) -> str:
    """libmoe_hostsan.so: every object as in build(), moe_api.cpp's host code
    with the sanitizers."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    # device objects of a build newer than every source are reused
    newest = max(os.path.getmtime(f) for f in glob.glob(os.path.join(CSRC, "*")))

    def obj(src: str) -> str:
        o = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
        if os.path.exists(o) and os.path.getmtime(o) >= newest:
            return o
        return _compile(src, verbose)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(obj, srcs))
    objs.append(_compile(os.path.join(CSRC, "moe_api.cpp"), verbose, HOST_SAN, ".hostsan.o"))
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC",
           "-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-shared-libsan",
           "-o", LIB_HOSTSAN, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    return LIB_HOSTSAN


if __name__ == "__main__":
    if "--host-sanitize" in sys.argv:
        print(build_hostsan(verbose="-v" in sys.argv))
    else:
        print(build(verbose="-v" in sys.argv))
