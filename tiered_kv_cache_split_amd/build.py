"""Builds librkv.so (all HIP kernels and the C-ABI runtime) for gfx950, in-tree.

Usage: ``python -m tiered_kv_cache_split_amd.build`` or ``build()`` from Python.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "librkv.so")
SOURCES = ["rkv_decode.hip", "rkv_decode_mma.hip", "rkv_decode_mma16.hip", "rkv_decode_hd.hip", "rkv_prefill.hip", "rkv_merge.hip", "rkv_aux.hip", "rkv_bcache.hip", "rkv_host_tail.cpp", "rkv_runtime.cpp"]
# host code only (the CPU tail partial): no device pass
HOST_ONLY = {"rkv_host_tail.cpp"}
ARCH = "gfx950"
# Packed FP32 instructions are disabled for all device code (their generated forms are
# avoided on this target); the host pass ignores the feature with a warning.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compile every source to an object (in parallel) and link librkv.so."""
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    cc = hipcc()
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src + ".o")
        objs.append(obj)
        lang = ["-x", "hip"] + (["--offload-host-only"] if src in HOST_ONLY else [])
        cmd = [cc, *lang, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-c",
               os.path.join(CSRC, src), "-o", obj, f"-I{INCLUDE}", f"-I{CSRC}", *DEVICE_FLAGS]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        if len([p for p in procs if p[1].poll() is None]) >= jobs:
            procs[0][1].wait()
    for src, p in procs:
        out, _ = p.communicate()
        text = "\n".join(l for l in out.decode(errors="replace").splitlines()
                         if "not a recognized feature" not in l and "--hip-link" not in l)
        if p.returncode != 0:
            raise RuntimeError(f"compiling {src} failed:\n{text}")
        if verbose and text.strip():
            print(text)
    tmp = LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking librkv.so failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
