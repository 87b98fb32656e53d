"""CPU oracle for the NVFP4 block-scaled GEMM -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  It shares no code, table or helper with
the HIP library in ``nvfp4_block_scaled_07_amd`` and never calls it.  Every
value is computed in numpy: fp64 for the contraction, fp32 where the quantiser
fixes fp32 operations.

Sources (the pages, by title and section):

* P1 = "The Moment the Zeros Disappeared: A Pivotal FP4 Kernel Test on
  Blackwell SM120".
* P2 = "The Art of Reading the Manual: Debugging FP4 GEMM Kernels on Blackwell
  SM120".
* P3 = "When a Benchmark Crashes: The Elusive FP4 GEMM Comparison on Blackwell
  SM120".

What the method computes (P2 "The Message": the ``mm_fp4`` signature with
``a, b, a_descale, b_descale, alpha, out_dtype=bfloat16, block_size=16``;
P3 "Input Knowledge Required" items 3 and 4; P1 "The Subject Message: A
Corrected Test"):

    D[m, n] = bf16( alpha * sum_k  xA[m, k] * xB[n, k] )
    xA[m, k] = E2M1(codeA[m, k]) * E4M3(sfA[m, k // 16])
    xB[n, k] = E2M1(codeB[n, k]) * E4M3(sfB[n, k // 16])

The products are exact and accumulated in fp64 here (P3 "Input Knowledge
Required" item 4: dequantise on the fly, multiply-accumulate in a higher
precision).  Readings taken where the pages are silent are marked READING.

Storage conventions:

* A is ``uint8[M][K/2]`` (two codes per byte, P2 "Assumptions and Their
  Consequences", P3 "Input Knowledge Required" item 3).
* B is the column-major K x N operand of P1 "The Subject Message" (item 3):
  K-contiguous, i.e. ``uint8[N][K/2]`` in memory.
* Scales are raw e4m3fn bytes (P1 "The Testing Journey": uint8 viewed as
  float8_e4m3fn), ``uint8[rows][K/16]`` row-major (READING: linear layout,
  the default ``use_8x4_sf_layout=False`` of P2 "The Message").
* READING (packing order): element 2j sits in bits 0-3 and element 2j+1 in
  bits 4-7 of byte j.

Parity pins for every function live in ``tests/test_oracle_*.py``.  One
part is "parity unpinned": the 128 x 4 tiled scale layout
(:func:`scales_to_128x4`, :func:`scales_from_128x4`) and the 8 x 4 one
(:func:`scales_to_8x4`, :func:`scales_from_8x4`) are readings of layouts the
pages only name; their tests check the index formulas against independent
restatements, which catches slips but not a wrong reading.
"""
from __future__ import annotations

import math

import numpy as np

BLOCK = 16            # P2 "Assumptions and Their Consequences": block_size = 16
E2M1_MAX = 6.0        # largest e2m1 magnitude (OCP MX v1.0 FP4 E2M1)
E4M3_MAX = 448.0      # largest finite e4m3fn magnitude (OCP OFP8 E4M3)


# ---------------------------------------------------------------------------
# Code tables, written from the element-format definitions.
# ---------------------------------------------------------------------------
def e2m1_value(code: int) -> float:
    """Value of a 4-bit e2m1 code: sign bit 3, exponent bits 2-1 (bias 1),
    mantissa bit 0; exponent 0 is subnormal (m * 0.5).  P3 "Input Knowledge
    Required" item 3 names the 4-bit float; the bit layout is the OCP MX v1.0
    FP4 E2M1 definition."""
    sign = -1.0 if code & 0x8 else 1.0
    e = (code >> 1) & 0x3
    m = code & 0x1
    mag = m * 0.5 if e == 0 else 2.0 ** (e - 1) * (1.0 + m / 2.0)
    return sign * mag


def e4m3_value(byte: int) -> float:
    """Value of an e4m3fn byte (P1 "The Testing Journey", P3 "Input Knowledge
    Required" item 3: float8_e4m3fn scales): sign bit 7, exponent bits 6-3
    (bias 7), mantissa bits 2-0; exponent 0 is subnormal m * 2**-9; 0x7F/0xFF
    are NaN; there is no infinity."""
    sign = -1.0 if byte & 0x80 else 1.0
    e = (byte >> 3) & 0xF
    m = byte & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return sign * m * 2.0 ** -9
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E2M1_LUT = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
E4M3_LUT = np.array([e4m3_value(b) for b in range(256)], dtype=np.float64)
# Non-negative finite e4m3 values in code order (codes 0x00..0x7E): increasing.
_E4M3_POS = E4M3_LUT[:0x7F].copy()
# Non-negative e2m1 magnitudes in code order (codes 0..7): increasing.
_E2M1_POS = E2M1_LUT[:8].copy()


# ---------------------------------------------------------------------------
# Rounding to the two formats.
# ---------------------------------------------------------------------------
def _nearest_even_code(mag: np.ndarray, grid: np.ndarray) -> np.ndarray:
    """Index of the grid value nearest to ``mag`` (>= 0, <= grid[-1]); a tie
    goes to the even index.  For both formats the low bit of the code is the
    low mantissa bit, so this is round-to-nearest-even."""
    mag = np.asarray(mag, dtype=np.float64)
    hi = np.searchsorted(grid, mag, side="left")      # grid[hi] >= mag
    hi = np.clip(hi, 0, len(grid) - 1)
    lo = np.clip(hi - 1, 0, len(grid) - 1)
    d_lo = mag - grid[lo]
    d_hi = grid[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    idx = np.where(pick_hi, hi, lo)
    return np.where(grid[hi] == mag, hi, idx).astype(np.uint8)


def e4m3_encode(t: np.ndarray) -> np.ndarray:
    """fp32 -> e4m3fn byte, round to nearest even, saturating to +-448
    (READING: the pages only say the scales are float8_e4m3fn, P3 "Input
    Knowledge Required" item 3).  Inputs must be finite."""
    t = np.asarray(t, dtype=np.float32).astype(np.float64)
    mag = np.minimum(np.abs(t), E4M3_MAX)
    code = _nearest_even_code(mag, _E4M3_POS)
    sign = np.where(np.signbit(t), 0x80, 0x00).astype(np.uint8)
    return (code | sign).astype(np.uint8)


def e2m1_encode(y: np.ndarray) -> np.ndarray:
    """fp32 -> e2m1 code, round to nearest even, saturating to +-6 (READING).
    The sign bit of ``y`` is kept, so a negative value that rounds to zero
    gives code 0x8 (it decodes to -0 and leaves D unchanged)."""
    y = np.asarray(y, dtype=np.float32).astype(np.float64)
    mag = np.minimum(np.abs(y), E2M1_MAX)
    code = _nearest_even_code(mag, _E2M1_POS)
    sign = np.where(np.signbit(y), 0x8, 0x0).astype(np.uint8)
    return (code | sign).astype(np.uint8)


# ---------------------------------------------------------------------------
# Quantisation (prologue) and the tensor-level scales.
# ---------------------------------------------------------------------------
def global_encode_scale(x: np.ndarray) -> np.float32:
    """Per-tensor encode scale gs = (6 * 448) / amax(|x|) in fp32; 1 if the
    tensor is all zero.  READING of the workload's "global scales by
    amax/(6*448), alpha = 1/(gsA*gsB)": amax/(6*448) is the decode factor
    1/gs, and alpha is the product of the two decode factors."""
    amax = np.float32(np.max(np.abs(np.asarray(x, dtype=np.float32)))) if np.size(x) else np.float32(0)
    if amax == 0:
        return np.float32(1.0)
    return np.float32(np.float32(E2M1_MAX * E4M3_MAX) / amax)


def alpha_from_scales(gs_a, gs_b) -> np.float32:
    """alpha = 1 / (gsA * gsB) in fp32 (P1 "The Subject Message": alpha is the
    scalar of the fused multiply-add; value per the reading above)."""
    return np.float32(np.float32(1.0) / (np.float32(gs_a) * np.float32(gs_b)))


def quantize(x: np.ndarray, gs=np.float32(1.0)):
    """fp32 ``[R][K]`` -> (packed codes ``uint8[R][K/2]``, scales ``uint8[R][K/16]``).

    Per 16-element block of one row (P2 "Assumptions and Their Consequences":
    block_size 16; READING for every arithmetic step, all in fp32 with
    round-to-nearest-even):

    1. amax_b = max |x| over the block;
    2. t = (amax_b / 6) * gs;   sf = e4m3_encode(t)  (saturating);
    3. r = gs / E4M3(sf)  (correctly rounded division), or 0 when E4M3(sf) = 0;
    4. y = x * r;   code = e2m1_encode(y);
    5. pack two codes per byte, element 2j in the low nibble.
    """
    x = np.asarray(x, dtype=np.float32)
    if x.ndim != 2 or x.shape[1] % BLOCK:
        raise ValueError("quantize expects [R][K] with K % 16 == 0")
    R, K = x.shape
    gs = np.float32(gs)
    xb = x.reshape(R, K // BLOCK, BLOCK)
    amax = np.max(np.abs(xb), axis=2) if R else np.zeros((0, K // BLOCK), np.float32)
    t = (amax / np.float32(6.0)).astype(np.float32) * gs
    sf = e4m3_encode(t)
    sv = E4M3_LUT[sf].astype(np.float32)
    r = np.zeros_like(sv)
    nz = sv != 0
    r[nz] = gs / sv[nz]
    y = (xb * r[:, :, None]).astype(np.float32)
    codes = e2m1_encode(y).reshape(R, K)
    q = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return q, sf.reshape(R, K // BLOCK)


# ---------------------------------------------------------------------------
# Dequantisation and the contraction.
# ---------------------------------------------------------------------------
def unpack_codes(q: np.ndarray) -> np.ndarray:
    """``uint8[R][K/2]`` -> ``uint8[R][K]`` codes (element 2j = low nibble)."""
    q = np.asarray(q, dtype=np.uint8)
    R, H = q.shape
    codes = np.empty((R, 2 * H), dtype=np.uint8)
    codes[:, 0::2] = q & 0xF
    codes[:, 1::2] = q >> 4
    return codes


def dequant(q: np.ndarray, sf: np.ndarray) -> np.ndarray:
    """x[r, k] = E2M1(code[r, k]) * E4M3(sf[r, k // 16]) in fp64 (exact: at
    most 6 significant bits)."""
    codes = unpack_codes(q)
    K = codes.shape[1]
    sf = np.asarray(sf, dtype=np.uint8)
    if sf.shape != (codes.shape[0], K // BLOCK):
        raise ValueError("scale shape does not match codes")
    return E2M1_LUT[codes] * np.repeat(E4M3_LUT[sf], BLOCK, axis=1)


def gemm_fp64(a, a_sf, b, b_sf) -> np.ndarray:
    """S[m, n] = sum_k xA[m, k] * xB[n, k] in fp64 (a library dgemm on the
    dequantised operands; B is K-contiguous ``[N][K/2]``)."""
    xa = dequant(a, a_sf)
    xb = dequant(b, b_sf)
    if xa.shape[1] != xb.shape[1]:
        raise ValueError("K mismatch")
    return xa @ xb.T


def bf16_rne(x: np.ndarray) -> np.ndarray:
    """fp64 -> bf16 bit patterns (uint16), round to nearest, ties to even,
    applied directly to the fp64 value (one rounding)."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.float64)
    mant, expo = np.frexp(x)                       # x = mant * 2**expo, |mant| in [0.5, 1)
    normal = np.abs(x) >= 2.0 ** -126
    # normal range: 8 significant bits
    out[normal] = np.ldexp(np.rint(np.ldexp(mant[normal], 8)), expo[normal] - 8)
    # subnormal range: quantum 2**-133
    sub = ~normal
    out[sub] = np.ldexp(np.rint(np.ldexp(x[sub], 133)), -133)
    big = np.abs(out) > 3.3895313892515355e38      # beyond the largest finite bf16
    out[big] = np.copysign(np.inf, out[big])
    nan = np.isnan(x)
    bits = (out.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    bits[nan] = 0x7FC0
    return bits


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def gemm(a, a_sf, b, b_sf, alpha=np.float32(1.0)) -> np.ndarray:
    """D = bf16(alpha * S) as uint16 bits (P2 "The Message": out_dtype
    bfloat16, optional alpha; alpha absent means 1)."""
    s = gemm_fp64(a, a_sf, b, b_sf)
    return bf16_rne(np.float64(np.float32(alpha)) * s)


def grouped_gemm(a, a_sf, b, b_sf, offsets, alpha, d_init) -> np.ndarray:
    """Grouped-by-expert GEMM (P3 "Why This Message Was Written": 256 experts,
    8 active per token, per-expert FP4 GEMMs; the interface is a READING).
    Rows offsets[e] .. offsets[e+1]-1 of A multiply expert e's B[e]
    (``[E][N][K/2]``) with alpha[e]; rows outside every range keep d_init."""
    d = np.array(d_init, dtype=np.uint16, copy=True)
    offsets = np.asarray(offsets, dtype=np.int64)
    E = len(offsets) - 1
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            al = np.float32(1.0) if alpha is None else np.float32(alpha[e])
            d[lo:hi] = gemm(a[lo:hi], a_sf[lo:hi], b[e], b_sf[e], al)
    return d


# ---------------------------------------------------------------------------
# Fused activation quantisation: the step before the grouped GEMM in an MoE
# layer (tokens routed to experts are gathered and quantised, then multiplied
# by each expert's weights; P3 "Why This Message Was Written": 256 experts, 8
# active per token).  Nothing new is computed: the gather is a row copy and
# the quantiser and grouped GEMM are the functions above.
# ---------------------------------------------------------------------------
def bf16_bits_to_f32(bits) -> np.ndarray:
    """bf16 bit patterns -> fp32 values (exact: bf16 is the top half of fp32)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def gather_rows(x: np.ndarray, row_token, rows: int) -> np.ndarray:
    """Row i of the result is x[row_token[i]] (x[i] when row_token is None).
    READING: a token outside [0, T) gives a zero row."""
    T = x.shape[0]
    tok = np.arange(rows) if row_token is None else np.asarray(row_token, dtype=np.int64)[:rows]
    out = np.zeros((rows,) + x.shape[1:], dtype=x.dtype)
    ok = (tok >= 0) & (tok < T)
    out[ok] = x[tok[ok]]
    return out


def grouped_gemm_fused(x_bits, row_token, gs, b, b_sf, offsets, alpha, d_init, rows: int) -> np.ndarray:
    """D = grouped_gemm(quantize(gather(bf16 x), gs), B, offsets, alpha):
    the grouped GEMM whose A rows are the routed tokens' activations
    (bf16 ``[T][K]``), quantised with one encode scale gs for all rows."""
    a32 = gather_rows(bf16_bits_to_f32(x_bits), row_token, rows)
    a, a_sf = quantize(a32, np.float32(gs))
    return grouped_gemm(a, a_sf, b, b_sf, offsets, alpha, d_init)


# ---------------------------------------------------------------------------
# Interop: the 128 x 4 tiled scale layout.  The pages only name the switch
# between scale layouts (P2 "The Message": use_8x4_sf_layout=False) and never
# describe one.  READING: the tiled layout used by the CUTLASS NVFP4 path:
# the [rows][K/16] scale matrix, padded with zeros to a multiple of 128 rows
# and 4 columns, is stored as 512-byte tiles of 128 rows x 4 columns, tiles
# in row-major order; inside a tile, the scale of row r and column c sits at
# byte (r % 32) * 16 + ((r % 128) // 32) * 4 + c % 4.
# ---------------------------------------------------------------------------
def tiled128x4_size(rows: int, K: int) -> int:
    return (-(-rows // 128) * 128) * (-(-(K // 16) // 4) * 4)


def scales_to_128x4(sf: np.ndarray) -> np.ndarray:
    """Linear ``uint8[rows][K/16]`` -> the 128 x 4 tiled byte sequence."""
    rows, cols = sf.shape
    tr, tc = -(-rows // 128), -(-cols // 4)
    out = np.zeros(tr * tc * 512, dtype=np.uint8)
    r = np.arange(rows)[:, None]
    c = np.arange(cols)[None, :]
    pos = ((r // 128) * tc + c // 4) * 512 + (r % 32) * 16 + ((r % 128) // 32) * 4 + c % 4
    out[pos] = sf
    return out


def scales_from_128x4(tiled: np.ndarray, rows: int, K: int) -> np.ndarray:
    """The 128 x 4 tiled byte sequence -> linear ``uint8[rows][K/16]``."""
    cols = K // 16
    tc = -(-cols // 4)
    r = np.arange(rows)[:, None]
    c = np.arange(cols)[None, :]
    pos = ((r // 128) * tc + c // 4) * 512 + (r % 32) * 16 + ((r % 128) // 32) * 4 + c % 4
    return np.asarray(tiled, dtype=np.uint8)[pos]


# The 8 x 4 layout: the other swizzled layout that the ``use_8x4_sf_layout``
# switch of P2 "The Message" names (the pages describe neither).  READING:
# the scale matrix, padded with zeros to a multiple of 8 rows and 4 columns,
# is stored as 32-byte tiles of 8 rows x 4 columns, tiles in row-major order;
# inside a tile, the scale of row r and column c sits at byte
# (r % 8) * 4 + c % 4.  Parity unpinned (a reading, as for the 128 x 4 one).
def tiled8x4_size(rows: int, K: int) -> int:
    return (-(-rows // 8) * 8) * (-(-(K // 16) // 4) * 4)


def _pos_8x4(rows: int, cols: int) -> np.ndarray:
    tc = -(-cols // 4)
    r = np.arange(rows)[:, None]
    c = np.arange(cols)[None, :]
    return ((r // 8) * tc + c // 4) * 32 + (r % 8) * 4 + c % 4


def scales_to_8x4(sf: np.ndarray) -> np.ndarray:
    """Linear ``uint8[rows][K/16]`` -> the 8 x 4 tiled byte sequence."""
    rows, cols = sf.shape
    out = np.zeros(tiled8x4_size(rows, 16 * cols), dtype=np.uint8)
    out[_pos_8x4(rows, cols)] = sf
    return out


def scales_from_8x4(tiled: np.ndarray, rows: int, K: int) -> np.ndarray:
    """The 8 x 4 tiled byte sequence -> linear ``uint8[rows][K/16]``."""
    return np.asarray(tiled, dtype=np.uint8)[_pos_8x4(rows, K // 16)]


# ---------------------------------------------------------------------------
# Exact integer mode (an independent check of the fp64 path).
# ---------------------------------------------------------------------------
def _int_tables():
    """E2M1 * 2 and E4M3 * 2**9 are integers for every finite code."""
    e2 = np.array([int(round(2 * v)) for v in E2M1_LUT], dtype=np.int64)
    fin = ~np.isnan(E4M3_LUT)
    e4 = np.zeros(256, dtype=np.int64)
    e4[fin] = np.round(E4M3_LUT[fin] * 512).astype(np.int64)
    return e2, e4, fin


def gemm_exact_int(a, a_sf, b, b_sf) -> np.ndarray:
    """S * 2**20 as an exact int64 sum (x * 2**10 is an integer below 2**22,
    so |S| * 2**20 < 2**56 for K <= 8192).  NaN scales are rejected."""
    e2, e4, fin = _int_tables()
    def _ints(q, sf):
        sf = np.asarray(sf, dtype=np.uint8)
        if not fin[sf].all():
            raise ValueError("NaN scale")
        return e2[unpack_codes(q)] * np.repeat(e4[sf], BLOCK, axis=1)
    ia, ib = _ints(a, a_sf), _ints(b, b_sf)
    if ia.shape[1] > 8192:
        raise ValueError("exact mode limited to K <= 8192")
    return ia @ ib.T


# ---------------------------------------------------------------------------
# Tolerance for a floating-point accumulator.
# ---------------------------------------------------------------------------
def bf16_ulp(bits: np.ndarray) -> np.ndarray:
    """ulp of a bf16 value: 2**(floor(log2|y|) - 7); 0 for y = 0."""
    y = np.abs(bf16_to_f64(bits))
    out = np.zeros_like(y)
    nz = y > 0
    out[nz] = np.ldexp(1.0, np.floor(np.log2(y[nz])).astype(np.int64) - 7)
    return out


def gemm_tolerance(a, a_sf, b, b_sf, alpha, d_ref_bits) -> np.ndarray:
    """Per-element bound |D - D_ref| <= 2 ulp_bf16(D_ref) + floor, with
    floor = 8 |alpha| sqrt(K) 2**-24 sqrt(sum_k (xA xB)**2): the bf16 bound of
    the target plus the probabilistic fp32 summation error (Higham-Mary,
    sqrt(K) u times the 2-norm of the terms), which no fp32 accumulator can
    avoid where the sum cancels."""
    return tolerance_dequantized(dequant(a, a_sf), dequant(b, b_sf), alpha, d_ref_bits)


def tolerance_dequantized(xa, xb, alpha, d_ref_bits) -> np.ndarray:
    """The bound of :func:`gemm_tolerance` from the dequantised operands
    ``xa [M][K]``, ``xb [N][K]`` (fp64)."""
    K = xa.shape[1]
    l2 = np.sqrt((xa * xa) @ (xb * xb).T)
    floor = 8.0 * abs(float(np.float32(alpha))) * math.sqrt(K) * 2.0 ** -24 * l2
    return 2.0 * bf16_ulp(d_ref_bits) + floor
