"""Compile libzha.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Usage: ``python -m hierarchical_tree_indexed_build_amd.build_lib``.
"""
from __future__ import annotations

import os
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libzha.so")
SOURCES = ["zha_abi.hip", "build.hip", "route.hip", "route_dense.hip", "attend.hip", "pseudo.hip"]
ARCH = os.environ.get("ZHA_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared",
    f"--offload-arch={ARCH}",
    # packed fp32 VALU forms are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden", "-Wall", "-Wno-unused-result",
    "-I", os.path.join(ROOT, "include"),
]


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compile every source to an object in parallel, then link libzha.so. Returns the library path."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    t0 = time.time()
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        objs.append(obj)
        cmd = [hipcc, *[f for f in FLAGS if f != "-shared"], "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        while sum(p.poll() is None for _, p in procs) >= jobs:
            time.sleep(0.05)
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        if p.returncode != 0:
            failed.append((src, out))
        elif verbose and out.strip():
            print(out, flush=True)
    if failed:
        msg = "\n".join(f"--- {s} ---\n{o}" for s, o in failed)
        raise RuntimeError(f"hipcc failed:\n{msg}")
    tmp = LIB + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} in {time.time() - t0:.1f}s", flush=True)
    return LIB


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
