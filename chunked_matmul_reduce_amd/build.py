"""Builds libmmar.so (the gfx950 kernels and the C ABI of include/mmar.h) in place.

    python chunked_matmul_reduce_amd/build.py       # from the repository root (a script:
                                                     # the package itself needs the library)

hipcc cross-compiles for gfx950 without a GPU.  Flags: -O3; -ffp-contract=off so that
no multiply-add in the epilogue is fused (the output bits must not depend on the
schedule); packed fp32 ops disabled in device code.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libmmar.so")
SOURCES = [os.path.join(PKG, "csrc", "tile_kernel.hip"), os.path.join(PKG, "csrc", "reduce_kernels.hip"),
           os.path.join(PKG, "csrc", "unfused.hip"), os.path.join(PKG, "csrc", "adam.hip"),
           os.path.join(PKG, "csrc", "noalloc.hip"), os.path.join(PKG, "csrc", "mmar.cpp")]
HEADERS = [os.path.join(PKG, "csrc", "mmar_internal.h"), os.path.join(PKG, "csrc", "device_common.h"),
           os.path.join(ROOT, "include", "mmar.h")]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmmar.so)")


def command(out: str) -> list:
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-result", "-I", os.path.join(ROOT, "include"),
            *SOURCES, "-o", out]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 target feature; that warning is noise
    noise = ("packed-fp32-ops", "is not a recognized feature for this target")
    err = "\n".join(ln for ln in r.stderr.splitlines() if not any(n in ln for n in noise))
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
