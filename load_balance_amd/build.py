"""Compiles the HIP sources under csrc/ into load_balance_amd/liblbattn.so for gfx950.

    python -m load_balance_amd.build

Each source is compiled to its own object under _build/ (in parallel), then the
objects are linked.  Every HIP source is compiled with packed fp32 arithmetic
disabled (-target-feature -packed-fp32-ops); hipcc's host pass warns that it
does not know that feature, which is harmless.
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
LIB = os.path.join(PKG, "liblbattn.so")
SOURCES = ["plan.hip", "attn_fwd.hip", "lse_merge.hip", "bwd.hip", "api.cpp"]
ARCH = os.environ.get("LB_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build liblbattn.so)")


COMMON = ["-O3", "-std=c++17", "-fPIC", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wno-unused-command-line-argument"]
# The attention kernel is scheduled with the iterative ILP strategy: the default one keeps
# a single LDS read in flight ahead of the QK^T MFMAs in its key loop.  Its atomics are all
# issued by one lane, and the atomic optimizer's wave-wide rewrite would make that lane wait
# for the result (and every load before it) at once instead of where it is used.
EXTRA = {"attn_fwd.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp",
                          "-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]}
OBJ_DIR = os.path.join(PKG, "_build")


def compile_command(src: str, obj: str) -> list[str]:
    return [hipcc(), "-x", "hip", f"--offload-arch={ARCH}", "-c"] + COMMON + EXTRA.get(src, []) + [
        "-I", os.path.join(ROOT, "include"), "-o", obj, os.path.join(CSRC, src)]


def link_command(objs: list[str], out: str) -> list[str]:
    return [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", out] + objs


def _run(cmd: list[str], verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    objs = [os.path.join(OBJ_DIR, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as pool:
        list(pool.map(lambda so: _run(compile_command(*so), verbose), zip(SOURCES, objs)))
    tmp = LIB + ".tmp"
    _run(link_command(objs, tmp), verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
