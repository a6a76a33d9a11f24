"""Build the gfx950 HIP library ``libpdrsplat.so`` in-tree with hipcc.

Flags: gfx950 only, -O3, packed-FP32 instruction selection disabled,
hardware fp32 atomics (``-munsafe-fp-atomics`` lets atomicAdd on float use
``global_atomic_add_f32``).
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SOURCES = ["csrc/bin.hip", "csrc/raster.hip", "csrc/loss.hip", "csrc/adapter.hip", "csrc/span.hip",
           "csrc/abi.hip",
           "csrc/timing.hip"]
LIB = os.path.join(PKG, "libpdrsplat.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-munsafe-fp-atomics",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    p = os.path.join(rocm, "bin", "hipcc")
    return p if os.path.exists(p) else "hipcc"


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"),
           *[os.path.join(PKG, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building %s" % LIB)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
