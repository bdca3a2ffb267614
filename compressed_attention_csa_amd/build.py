"""Build libcsa.so (the HIP kernels and the C ABI) in-tree for gfx950.

Usage: python -m compressed_attention_csa_amd.build [--debug]   (or call build()).
Every source is compiled to an object under _build/ in parallel, then linked.
build(debug=True) makes libcsa_debug.so instead, compiled with CSA_DEBUG: it
poisons workspace scratch and LDS with NaN words before use and checks launch
plans on the host (the same kernels otherwise).
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libcsa.so")
DEBUG_LIB = os.path.join(PKG, "libcsa_debug.so")
SOURCES = ["compress.hip", "index.hip", "index_prefill.hip", "attend.hip", "api.cpp", "profile.cpp",
           "noalloc.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
    # Packed fp32 instructions are kept out of generated code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result", "-I", os.path.join(ROOT, "include"),
]


def _compile(src: str, debug: bool = False) -> str:
    obj = os.path.join(BUILD, "debug" if debug else "", src + ".o")
    lang = [] if src.endswith(".hip") else ["-x", "hip"]
    cmd = [HIPCC, *FLAGS, *(["-DCSA_DEBUG=1"] if debug else []), *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, debug: bool = False) -> str:
    os.makedirs(os.path.join(BUILD, "debug"), exist_ok=True)
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, debug), srcs))
    out = DEBUG_LIB if debug else LIB
    tmp = out + ".tmp"
    cmd = [HIPCC, "-shared", "--offload-arch=gfx950", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print("built", out)
    return out


if __name__ == "__main__":
    build(verbose=True, debug="--debug" in sys.argv[1:])
    sys.exit(0)
