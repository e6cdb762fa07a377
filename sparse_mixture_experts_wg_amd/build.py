"""Build libmoe.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

    python sparse_mixture_experts_wg_amd/build.py

Objects go to sparse_mixture_experts_wg_amd/_build/, the library to
sparse_mixture_experts_wg_amd/libmoe.so (both in-tree, both git-ignored).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIBRARY = os.path.join(PKG, "libmoe.so")

ARCH = "gfx950"
SOURCES = ["abi.cpp", "noalloc.hip", "norm.hip", "route.hip", "permute.hip", "combine.hip", "gemm_f32.hip",
           "gemm_stream.hip", "gemm_tiled.hip"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmoe.so)")


def _flags(debug: bool = False):
    f = ["-std=c++17", "-fPIC", "-Wall", f"-I{INCLUDE}", f"-I{CSRC}",
         # no packed fp32 instructions anywhere in the device code
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    f += ["-O0", "-g"] if debug else ["-O3"]
    return f


def _compile(src: str, debug: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    path = os.path.join(CSRC, src)
    cmd = [hipcc()] + _flags(debug)
    if src.endswith(".hip"):
        cmd += ["-x", "hip", f"--offload-arch={ARCH}"]
    cmd += ["-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{msgs}")
    return obj


def build(debug: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max(1, min(jobs, len(SOURCES)))) as ex:
        objs = list(ex.map(lambda s: _compile(s, debug), SOURCES))
    tmp = LIBRARY + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build(debug="--debug" in sys.argv))
