"""Compile libskv.so (the HIP kernels and the C ABI of include/skv.h) for gfx950, in tree.

Usage: python streaming_kv_cache_write_amd/build.py   (a script: importing the package would
load the library that this script compiles).
Every call recompiles; objects go to _build/ beside this file, the library to libskv.so.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libskv.so")
SOURCES = ["api.hip", "kv_write.hip", "kv_rope.hip", "attn_f32.hip", "attn_flash.hip", "attn_decode.hip",
           "peaks.hip"]
ARCH = os.environ.get("SKV_OFFLOAD_ARCH", "gfx950")

# -packed-fp32-ops: keep the compiler from forming packed fp32 arithmetic (the kernels use
# scalar fp32 math only).
FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + os.path.join(os.path.dirname(HERE), "include")]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libskv)")


# A second library for the host-side checks under AddressSanitizer: the C ABI's host code
# (argument validation, dispatch, launch configuration) instrumented, the device code and the
# other sources as in the product. Only the CPU ABI tests load it (they launch no kernel).
ASAN_LIB = os.path.join(BUILD_DIR, "libskv_asan.so")
ASAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
              "-Xarch_host", "-fsanitize-recover=address"]


def asan_runtime() -> str:
    """The clang ASan runtime that must be preloaded into a process loading ASAN_LIB."""
    llvm = os.path.join(os.path.dirname(os.path.dirname(_hipcc())), "llvm", "lib", "clang")
    for ver in sorted(os.listdir(llvm), reverse=True) if os.path.isdir(llvm) else []:
        p = os.path.join(llvm, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(p):
            return p
    raise RuntimeError("clang ASan runtime not found")


def _compile(src: str, extra=(), suffix: str = "") -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + suffix + ".o")
    cmd = [_hipcc(), *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, out: str, extra=()) -> None:
    tmp = out + ".tmp"
    cmd = [_hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", *extra, *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking {out} failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES) + 1)) as ex:
        objs_f = [ex.submit(_compile, s) for s in SOURCES]
        asan_f = ex.submit(_compile, "api.hip", ASAN_FLAGS, "_asan")
        objs = [f.result() for f in objs_f]
        asan_api = asan_f.result()
    _link(objs, LIB)
    _link([asan_api] + [o for o in objs if not o.endswith(os.sep + "api.o")], ASAN_LIB,
          ["-Xarch_host", "-fsanitize=address", "-shared-libasan"])
    if verbose:
        print("built", LIB, "and", ASAN_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
