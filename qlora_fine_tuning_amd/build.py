"""Builds the gfx950 HIP library libqlora_mi355x.so in-tree with hipcc.

Usage: python -m qlora_fine_tuning_amd.build   (or call build()).
Every call recompiles; objects go to <repo>/_build/, the library next to
this file so that it travels with the source tree.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libqlora_mi355x.so")
SOURCES = ["nf4.hip", "w16.hip", "gemm.hip", "lora.hip", "probe.hip", "fast.hip", "scratch.hip", "api.cpp"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def common_flags():
    return [
        "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
        "-Wall", "-Wno-unused-function", "-Wno-pass-failed",
        # packed fp32 VALU ops are kept out of all device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"),
    ]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + common_flags() + ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


def build_host_sanitized(verbose: bool = True) -> str:
    """A copy of the library whose host code (csrc/api.cpp: argument checks,
    workspace carving, stream and event handling) is built by g++ with
    AddressSanitizer and UndefinedBehaviorSanitizer. The kernels' objects are
    the ones build() made, unchanged (no GPU code is instrumented). Load it
    with QLORA_LIB_PATH=<path> and the ASan runtime preloaded."""
    if not all(os.path.exists(os.path.join(BUILD, os.path.splitext(s)[0] + ".o")) for s in SOURCES):
        build(verbose=False)
    out = os.path.join(BUILD, "san")
    os.makedirs(out, exist_ok=True)
    api_o = os.path.join(out, "api.o")
    cc = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-fno-omit-frame-pointer",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
          "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
          "-c", os.path.join(CSRC, "api.cpp"), "-o", api_o]
    res = subprocess.run(cc, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"g++ (sanitized api.cpp) failed:\n{res.stderr}")
    lib = os.path.join(out, "libqlora_mi355x.so")
    objs = [os.path.join(BUILD, os.path.splitext(s)[0] + ".o") for s in SOURCES if s != "api.cpp"]
    link = ["g++", "-shared", "-fsanitize=address,undefined", "-o", lib, api_o] + objs + [
        "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"]
    res = subprocess.run(link, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link (sanitized) failed:\n{res.stderr}")
    if verbose:
        print("built", lib)
    return lib


if __name__ == "__main__":
    build()
