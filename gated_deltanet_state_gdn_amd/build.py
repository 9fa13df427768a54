"""Build the gfx950 HIP library ``libgdn.so`` in-tree (hipcc, no JIT cache).

    python -m gated_deltanet_state_gdn_amd.build [--jobs N]
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libgdn.so")
SOURCES = ["gdn_api.hip", "gdn_chunk_ws.hip", "gdn_relerr.hip", "gdn_adaptive.hip", "gdn_segment.hip"]
ARCH = os.environ.get("GDN_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for c in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"),
              shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def flags() -> list:
    return ["--offload-arch=" + ARCH, "-O3", "-fPIC", "-std=c++17",
            # packed fp32 ops off: ordinary float code only
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + flags() + ["-c", os.path.join(CSRC, src), "-o", obj]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        sys.stderr.write(p.stdout + p.stderr)
        raise RuntimeError("hipcc failed on " + src)
    return obj


def build(jobs: int = 4, verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


# Host-side sanitizers for the argument validation in gdn_api.hip: only host code is
# instrumented (each -fsanitize= follows -Xarch_host); device code is built as usual.
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined",
                 "-Xarch_host", "-fno-omit-frame-pointer"]


def build_host_sanitized(out_dir: str = os.path.join(BUILD, "hostsan")) -> str:
    """libgdn with an ASan+UBSan-instrumented gdn_api.hip, for CPU-only validation tests.

    The process that loads it must preload clang's ASan runtime
    (``clang_asan_runtime()``).  The other objects are the regular build's.
    """
    os.makedirs(out_dir, exist_ok=True)
    objs = []
    for src in SOURCES:
        if src == "gdn_api.hip":
            continue
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        if not os.path.exists(obj) or os.path.getmtime(obj) < os.path.getmtime(os.path.join(CSRC, src)):
            os.makedirs(BUILD, exist_ok=True)
            _compile(src)
        objs.append(obj)
    api = os.path.join(out_dir, "gdn_api.o")
    subprocess.check_call([hipcc()] + flags() + HOST_SANITIZE +
                          ["-c", os.path.join(CSRC, "gdn_api.hip"), "-o", api])
    lib = os.path.join(out_dir, "libgdn_hostsan.so")
    subprocess.check_call([hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", lib, api] + objs)
    return lib


def clang_asan_runtime() -> str:
    """Path of the ROCm clang's shared ASan runtime (includes the UBSan handlers)."""
    root = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm", "lib", "clang")
    for ver in sorted(os.listdir(root), reverse=True):
        p = os.path.join(root, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(p):
            return p
    raise RuntimeError("clang ASan runtime not found under " + root)


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=4)
    build(ap.parse_args().jobs)
