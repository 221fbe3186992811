"""Builds libfa.so (the HIP kernels and their C ABI) for gfx950 with hipcc.

The library is built in-tree, next to this file, so that it travels with the
source tree. ``build()`` always recompiles.
"""

from __future__ import annotations

import os
import shutil
import subprocess

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
LIB_PATH = os.path.join(PKG_DIR, "libfa.so")
SOURCES = [os.path.join(PKG_DIR, "csrc", "fa_fwd.hip"), os.path.join(PKG_DIR, "csrc", "fa_bwd.hip")]
HEADERS = [os.path.join(ROOT, "include", "fa.h"), os.path.join(PKG_DIR, "csrc", "fa_kernels.h"),
           os.path.join(PKG_DIR, "csrc", "fa_host.h")]

# -packed-fp32-ops: keep hipcc from emitting packed fp32 VALU instructions.
HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libfa.so")


def build(verbose: bool = False) -> str:
    """Compile every source into libfa.so; returns its path."""
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), "-o", tmp, *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def is_built() -> bool:
    return os.path.exists(LIB_PATH)


if __name__ == "__main__":
    print(build(verbose=True))
