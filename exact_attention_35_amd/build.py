"""Build libfa.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Usage: python -m exact_attention_35_amd.build
The library is written next to this file so that it travels with the source
tree; objects go to _build/ at the repository root.
"""

from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfa.so")
CALLER = os.path.join(PKG, "fa_c_caller")
SOURCES = ["fa_fwd.hip", "fa_bwd.hip", "fa_fp8.hip", "fa_api.cpp"]
ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # keep the compiler from forming packed fp32 instructions (v_pk_fma_f32 and friends)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE,
    "-I", CSRC,
]


def _hipcc() -> str:
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *COMMON_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd = [_hipcc(), *COMMON_FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    if out.strip():
        sys.stderr.write(out + "\n")
    return obj


def build(verbose: bool = True) -> str:
    """Compile every source for gfx950 and link libfa.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link of libfa.so failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, LIB)
    # a plain C-ABI caller (host code only, linked against libfa.so next to it)
    cmd = [_hipcc(), "-O2", "-std=c++17", "-Wall", "-I", INCLUDE, os.path.join(CSRC, "fa_c_caller.cpp"),
           "-L", PKG, "-lfa", "-Wl,-rpath,$ORIGIN", "-o", CALLER]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("build of fa_c_caller failed:\n" + res.stdout + res.stderr)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
