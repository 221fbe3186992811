"""Builds libfa.so (the HIP kernels and their C ABI) for gfx950 with hipcc.

The library is built in-tree, next to this file, so that it travels with the
source tree. ``build()`` always recompiles. It also builds libfa_sync.so, the
same sources with FA_SYNC_CHECK: every wait drains all copies and every
barrier is a full one, for the GPU test that compares the two builds' results
bit for bit (a race check). The sources compile in parallel.
"""

from __future__ import annotations

import os
import shutil
import subprocess

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
LIB_PATH = os.path.join(PKG_DIR, "libfa.so")
SYNC_LIB_PATH = os.path.join(PKG_DIR, "libfa_sync.so")
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


def _run_all(cmds, verbose):
    procs = []
    for cmd in cmds:
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
    errors = []
    for cmd, p in procs:
        out, err = p.communicate()
        if p.returncode != 0:
            errors.append(f"{' '.join(cmd)}\n({p.returncode}):\n{out}\n{err}")
    if errors:
        raise RuntimeError("hipcc failed:\n" + "\n".join(errors))


def build(verbose: bool = False) -> str:
    """Compile every source into libfa.so (and libfa_sync.so); returns the
    path of libfa.so."""
    obj_dir = os.path.join(PKG_DIR, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    common = [hipcc(), *[f for f in HIPCC_FLAGS if f != "-shared"], "-I", os.path.join(ROOT, "include")]
    objs = {LIB_PATH: [], SYNC_LIB_PATH: []}
    compiles = []
    for src in SOURCES:
        stem = os.path.splitext(os.path.basename(src))[0]
        for lib, extra, tag in ((LIB_PATH, [], ""), (SYNC_LIB_PATH, ["-DFA_SYNC_CHECK"], "_sync")):
            obj = os.path.join(obj_dir, f"{stem}{tag}.o")
            compiles.append([*common, *extra, "-c", "-o", obj, src])
            objs[lib].append(obj)
    _run_all(compiles, verbose)
    links = []
    for lib, files in objs.items():
        links.append([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", lib + ".tmp", *files])
    _run_all(links, verbose)
    for lib in objs:
        os.replace(lib + ".tmp", lib)
    return LIB_PATH


def is_built() -> bool:
    return os.path.exists(LIB_PATH)


if __name__ == "__main__":
    print(build(verbose=True))
