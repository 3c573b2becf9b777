"""Builds libqwen2_mi355x.so in-tree with hipcc for gfx950.

    python -m qwen2_decoder_forward_amd.build        (or build.build())
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(ROOT, "_build", "obj")
LIB = os.path.join(PKG, "libqwen2_mi355x.so")

SOURCES = ["k_gemv.hip", "k_attn.hip", "k_gemm.hip", "k_misc.hip", "k_probe.hip", "k_debug.hip",
           "qwen2_abi.cpp",
           "validate.cpp"]
ARCH = "gfx950"
# Packed-f32 VALU ops are disabled for every device pass; the compiler then
# emits scalar f32 arithmetic only.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
CFLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
          "-Wno-unused-function", "-I", os.path.join(ROOT, "include")]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the MI355X library cannot be built")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{out}")
    if out.strip() and verbose:
        print(out)


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    cc = hipcc()
    jobs = []
    for src in SOURCES:
        obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
        cmd = [cc] + CFLAGS + (DEVICE_FLAGS if src.endswith(".hip") else []) + [
            "-c", os.path.join(CSRC, src), "-o", obj]
        jobs.append((cmd, obj))
    with cf.ThreadPoolExecutor(min(8, len(jobs))) as ex:
        list(ex.map(lambda j: _run(j[0], verbose), jobs))
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + [o for _, o in jobs],
         verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
