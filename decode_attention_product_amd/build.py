"""Builds the HIP library libpqattn.so in-tree for gfx950.

    python -m decode_attention_product_amd.build

Every call compiles from source.  The packed-FP32 instruction family is
switched off for the device code (``-packed-fp32-ops``); the host pass warns
that it does not know that feature, which is harmless.
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
LIB = os.path.join(PKG, "libpqattn.so")

SOURCES = ["api.hip", "plan.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; the ROCm toolchain is needed to build libpqattn.so")
    return exe


def compile_flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}"]


def build(verbose: bool = False) -> str:
    """Compile libpqattn.so; returns its path.  Raises on a compiler error."""
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *compile_flags(), "-shared", "-o", tmp,
           *[os.path.join(CSRC, s) for s in SOURCES]]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
