"""Build the gfx950 shared library ``libnvfp4_gfx950.so`` in-tree with hipcc.

Run ``python -m nvfp4_block_scaled_07_amd.build`` (or call :func:`build`).
The quantiser needs IEEE fp32 semantics, so there is no fast-math, fp
contraction is off and fp32 division stays correctly rounded.  Packed fp32
instructions are disabled for all device code.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libnvfp4_gfx950.so")
SOURCES = ["api.hip", "gemm.hip", "layout.hip", "moe.hip", "quantize.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-ffp-contract=off", "-fno-fast-math", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
]


def command(out: str = LIB) -> list:
    return [HIPCC, *FLAGS, *[os.path.join(CSRC, s) for s in SOURCES], "-o", out]


def build(verbose: bool = False) -> str:
    """Compile every HIP source into the in-tree library; returns its path."""
    tmp = LIB + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass warns about the device-only target feature; that is harmless
    msgs = [l for l in (res.stdout + res.stderr).splitlines()
            if l.strip() and "packed-fp32-ops" not in l and "is not a recognized feature" not in l]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
