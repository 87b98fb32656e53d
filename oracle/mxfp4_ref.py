"""CPU oracle for the MXFP4 GEMM -- TEST INFRASTRUCTURE ONLY.

Only the test suite and ``bench.py`` may import this module.  It shares no
code with the HIP library and never calls it; numpy, fp64 for the contraction.

What is computed.  The ``mm_fp4`` signature the pages print has a
``use_nvfp4`` switch (P2 = "The Art of Reading the Manual: Debugging FP4 GEMM
Kernels on Blackwell SM120", section "The Message"); with it off the kernel
takes the MX format, which the pages do not describe further.  The format is
taken from the OCP Microscaling Formats (MX) specification v1.0, MXFP4:

* elements are FP4 E2M1 (the same element type as NVFP4, decoded by
  ``nvfp4_ref.e2m1_value``), two per byte, element 2j in the low nibble;
* every block of 32 consecutive elements along K shares one scale of type
  E8M0: an unsigned biased exponent, value 2**(byte - 127), byte 0xFF = NaN;
* x[r, k] = E2M1(code[r, k]) * 2**(sf[r, k // 32] - 127).

    D[m, n] = bf16( alpha * sum_k  xA[m, k] * xB[n, k] )

with A ``uint8[M][K/2]``, B the K-contiguous ``uint8[N][K/2]`` operand and
scales ``uint8[rows][K/32]`` (the same conventions as the NVFP4 oracle).
READING: the output type, alpha and the operand layout follow the NVFP4 call
of the same signature; only the scale type and block size change.

Each x is exact in fp64 (at most 2 significant bits, exponent within fp64's
range), so the fp64 products are exact and the sum is rounded once per
addition in fp64, far below the bf16 output step.
"""
from __future__ import annotations

import math

import numpy as np

from . import nvfp4_ref as nv

BLOCK = 32            # OCP MX v1.0: MXFP4 block size
E8M0_BIAS = 127
E8M0_NAN = 0xFF


def e8m0_value(byte: int) -> float:
    """E8M0 scale: 2**(byte - 127); 0xFF is NaN (OCP MX v1.0, E8M0)."""
    byte = int(byte)
    if not 0 <= byte <= 255:
        raise ValueError("byte out of range")
    if byte == E8M0_NAN:
        return math.nan
    return math.ldexp(1.0, byte - E8M0_BIAS)


E8M0_LUT = np.array([e8m0_value(b) for b in range(256)], dtype=np.float64)


def dequant(q: np.ndarray, sf: np.ndarray) -> np.ndarray:
    """x[r, k] = E2M1(code[r, k]) * 2**(sf[r, k // 32] - 127) in fp64."""
    codes = nv.unpack_codes(q)
    K = codes.shape[1]
    sf = np.asarray(sf, dtype=np.uint8)
    if K % BLOCK or sf.shape != (codes.shape[0], K // BLOCK):
        raise ValueError("scale shape does not match codes")
    return nv.E2M1_LUT[codes] * np.repeat(E8M0_LUT[sf], BLOCK, axis=1)


def gemm_fp64(a, a_sf, b, b_sf) -> np.ndarray:
    """S[m, n] = sum_k xA[m, k] * xB[n, k] in fp64 (a library dgemm on the
    dequantised operands)."""
    xa = dequant(a, a_sf)
    xb = dequant(b, b_sf)
    if xa.shape[1] != xb.shape[1]:
        raise ValueError("K mismatch")
    return xa @ xb.T


def gemm(a, a_sf, b, b_sf, alpha=np.float32(1.0)) -> np.ndarray:
    """D = bf16(alpha * S) as uint16 bit patterns (one rounding from fp64)."""
    return nv.bf16_rne(np.float64(np.float32(alpha)) * gemm_fp64(a, a_sf, b, b_sf))


def gemm_exact_int(a, a_sf, b, b_sf, e_min: int) -> np.ndarray:
    """S * 2**(2 - 2 e_min) as an exact Python-int matrix, for scale bytes
    >= e_min (2 E2M1 is an integer and 2**(byte - e_min) is one too); an
    independent route to S for small shapes."""
    e2 = [int(round(2 * v)) for v in nv.E2M1_LUT]
    ca, cb = nv.unpack_codes(a), nv.unpack_codes(b)
    sa, sb = np.asarray(a_sf, dtype=np.int64), np.asarray(b_sf, dtype=np.int64)
    if (sa < e_min).any() or (sb < e_min).any() or (sa == E8M0_NAN).any() or (sb == E8M0_NAN).any():
        raise ValueError("scale below e_min or NaN")
    M, K = ca.shape
    N = cb.shape[0]
    out = [[0] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            acc = 0
            for k in range(K):
                acc += (e2[ca[m, k]] << int(sa[m, k // BLOCK] - e_min)) * (e2[cb[n, k]] << int(sb[n, k // BLOCK] - e_min))
            out[m][n] = acc
    return out


def gemm_tolerance(a, a_sf, b, b_sf, alpha, d_ref_bits) -> np.ndarray:
    """Per-element bound: 2 bf16 ulps of the reference plus the probabilistic
    fp32 summation error 8 |alpha| sqrt(K) 2**-24 ||(xA xB)_k||_2, the same
    form as the NVFP4 bound (the hardware accumulates in fp32)."""
    return nv.tolerance_dequantized(dequant(a, a_sf), dequant(b, b_sf), alpha, d_ref_bits)
