"""Build the gfx950 shared library ``libnvfp4_gfx950.so`` in-tree with hipcc.

Run ``python -m nvfp4_block_scaled_07_amd.build`` (or call :func:`build`).
The quantiser needs IEEE fp32 semantics, so there is no fast-math, fp
contraction is off and fp32 division stays correctly rounded.  Packed fp32
instructions are disabled for all device code.  ``gemm_large.hip`` (the two
large-M NVFP4 tiles) is compiled first, to an object of its own, with the
iterative ILP instruction scheduler; the rest is compiled and linked with it
in one hipcc call.
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libnvfp4_gfx950.so")
SOURCES = ["api.hip", "gemm.hip", "layout.hip", "moe.hip", "quantize.hip"]
# sources compiled separately, with extra flags
SCHED_SOURCES = {"gemm_large.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"]}
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-ffp-contract=off", "-fno-fast-math", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
]


def object_commands(objdir: str) -> list:
    """hipcc calls that compile each of SCHED_SOURCES to an object in objdir."""
    flags = [f for f in FLAGS if f != "-shared"]
    return [[HIPCC, *flags, *extra, "-c", os.path.join(CSRC, src),
             "-o", os.path.join(objdir, os.path.splitext(src)[0] + ".o")]
            for src, extra in SCHED_SOURCES.items()]


def command(out: str = LIB, objdir: str = "") -> list:
    objs = [os.path.join(objdir, os.path.splitext(s)[0] + ".o") for s in SCHED_SOURCES]
    # "-x none": the objects are linked, not compiled as HIP
    return [HIPCC, *FLAGS, *[os.path.join(CSRC, s) for s in SOURCES], "-x", "none", *objs, "-o", out]


def _run(cmd: list, verbose: bool) -> None:
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


def build(verbose: bool = False) -> str:
    """Compile every HIP source into the in-tree library; returns its path."""
    tmp = LIB + ".tmp"
    with tempfile.TemporaryDirectory(prefix="nvfp4_build_") as objdir:
        for cmd in object_commands(objdir):
            _run(cmd, verbose)
        _run(command(tmp, objdir), verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
