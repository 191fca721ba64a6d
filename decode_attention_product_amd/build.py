"""Builds the HIP library libpqattn.so in-tree for gfx950.

    python -m decode_attention_product_amd.build

Every call compiles from source (one object per translation unit, in
parallel, under _build/, then one link).  The packed-FP32 instruction family is
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

SOURCES = ["api.hip", "api_fp8.hip", "plan.cpp"]
# the benchmark's read-only streaming reference, a library of its own
BENCH_SOURCES = ["stream_ref.hip"]
BENCH_LIB = os.path.join(PKG, "libpqbench.so")
ARCH = "gfx950"
BUILD_DIR = os.path.join(PKG, "_build")


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; the ROCm toolchain is needed to build libpqattn.so")
    return exe


def compile_flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}"]


_NOISE = "is not a recognized feature for this target"


def _clean(stderr: str) -> str:
    return "\n".join(l for l in stderr.splitlines() if _NOISE not in l)


def build(verbose: bool = False) -> str:
    """Compile libpqattn.so (and the benchmark's libpqbench.so); returns the
    path of libpqattn.so.  Raises on a compiler error.  The translation units
    compile in parallel, then each library links."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs, procs = [], []
    for src in SOURCES + BENCH_SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        cmd = [hipcc(), *compile_flags(), "-c", "-o", obj, os.path.join(CSRC, src)]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE,
                                            text=True)))
        objs.append(obj)
    failed = []
    for src, pr in procs:
        _, err = pr.communicate()
        err = _clean(err)
        if pr.returncode != 0:
            failed.append(f"{src} ({pr.returncode}):\n{err}")
        elif verbose and err.strip():
            print(err, file=sys.stderr)
    if failed:
        raise RuntimeError("hipcc failed: " + "\n".join(failed))
    n = len(SOURCES)
    for lib, lib_objs in ((LIB, objs[:n]), (BENCH_LIB, objs[n:])):
        tmp = lib + ".tmp"
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-o", tmp, *lib_objs]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed ({r.returncode}):\n{_clean(r.stderr)}")
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
