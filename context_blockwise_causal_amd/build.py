"""Builds libringattn.so in-tree with hipcc for gfx950.

Usage: ``python -m context_blockwise_causal_amd.build`` (or ``__graft_entry__.build()``).
Every source is compiled on each call; objects go to ``_build/`` and the shared library to
``context_blockwise_causal_amd/libringattn.so``.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libringattn.so")

SOURCES = ["ra_plan.cpp", "ra_host.cpp", "kern_rowops.hip", "kern_fwd.hip", "kern_bwd.hip",
           "kern_f32.hip", "ra_scratch.hip"]

ARCH = os.environ.get("RA_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC)")


def common_flags():
    return ["-O3", "-fPIC", "-std=c++17", f"-I{INCLUDE}", f"-I{CSRC}", "-Wall",
            "-Wno-unused-function"]


def compile_one(src: str) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD, src + ".o")
    if src.endswith(".hip"):
        cmd = [hipcc(), "-x", "hip", f"--offload-arch={ARCH}", "-munsafe-fp-atomics",
               # packed fp32 VALU forms are kept out of the generated code
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               *common_flags(), "-c", path, "-o", obj]
    else:
        cmd = [hipcc(), "-x", "c++", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", *common_flags(), "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{' '.join(cmd)}\n{out}")
    if out.strip():
        print(out, file=sys.stderr)
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed\n{' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
