"""Compile the HIP library ``libtpmlp.so`` for gfx950 with hipcc (in-tree).

Objects go to ``_build/`` at the repository root, the shared library next to this
file.  Every call recompiles every source.
"""
from __future__ import annotations

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libtpmlp.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)

SOURCES = ["api.cpp", "api_proj.cpp", "api_moe.cpp", "k_pack.hip", "k_stream.hip", "k_tiled.hip", "k_gemm.hip", "k_group.hip", "k_f32.hip", "k_reduce.hip",
           "k_quant.hip"]
ARCH = "gfx950"
# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU instructions.
HIP_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I" + os.path.join(ROOT, "include")]


def hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found; the ROCm toolchain is required to build libtpmlp")
    return p


def _compile(src: str) -> str:
    obj = os.path.join(OBJ_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + HIP_FLAGS + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("compiling %s failed:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def build(jobs: int = 8, verbose: bool = False) -> str:
    """Compile all sources and link ``libtpmlp.so``; returns its path."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=max(1, min(jobs, len(SOURCES)))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("linking %s failed:\n%s" % (LIB_NAME, r.stderr))
    os.replace(tmp, LIB_PATH)
    if verbose:
        print("built", LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
