"""CPU oracle for the MoE expert FFN around the NVFP4 grouped GEMM -- TEST
INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  It shares nothing with the HIP library
and never calls it; it builds on the NVFP4 oracle (``nvfp4_ref``) for the
quantiser and the grouped GEMM.

Source: P3 = "When a Benchmark Crashes: The Elusive FP4 GEMM Comparison on
Blackwell SM120", sections "Why This Message Was Written" (256 experts, 8
active per token, hidden size 6144, expert intermediate size 2048) and "The
Thinking Process Visible in Reasoning Parts" (the experts run through a fused
MoE kernel, cutlass_moe).  The pages do not describe the expert FFN beyond
that; the readings below are the plainest ones for that model family.

* READING (activation): SwiGLU, h = silu(gate) * up, silu(g) = g / (1 +
  exp(-g)); gate is the first I columns of the gate/up GEMM output, up the
  last I.
* READING (decision precision): the kernel forms h in fp32 and quantises it;
  the oracle evaluates h exactly (fp64) and rounds it once to fp32 before the
  quantiser.  exp is not correctly rounded in fp32 on the GPU, so the two h
  may differ by a few fp32 ulps; ``swiglu_quantize_bounds`` gives the codes a
  relative change of 2**-20 either way would produce, and tests accept either
  where a block is that close to a rounding boundary.
* READING (combine): out[t] = bf16( sum_j weight[t][j] * down[rows_of[t][j]] )
  (exact sum here); an index outside [0, rows) adds nothing.
"""
from __future__ import annotations

import numpy as np

from oracle import nvfp4_ref as o


def silu(g) -> np.ndarray:
    """g / (1 + exp(-g)) in fp64 (exp(-g) overflowing to inf gives -0)."""
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def swiglu(gu_bits: np.ndarray, I: int) -> np.ndarray:
    """h = silu(gate) * up in fp64 from bf16 gate/up ``[rows][2I]``."""
    gu = o.bf16_to_f64(gu_bits)
    return silu(gu[:, :I]) * gu[:, I:2 * I]


def swiglu_quantize(gu_bits: np.ndarray, I: int, gs=np.float32(1.0)):
    """NVFP4 codes and scales of h rounded once to fp32."""
    return o.quantize(swiglu(gu_bits, I).astype(np.float32), np.float32(gs))


def swiglu_quantize_bounds(gu_bits: np.ndarray, I: int, gs=np.float32(1.0), rel: float = 2.0 ** -20):
    """Quantisations of h * (1 - rel) and h * (1 + rel) (each rounded once to
    fp32): where both equal ``swiglu_quantize``, the codes are unique."""
    h = swiglu(gu_bits, I)
    lo = o.quantize((h * (1.0 - rel)).astype(np.float32), np.float32(gs))
    hi = o.quantize((h * (1.0 + rel)).astype(np.float32), np.float32(gs))
    return lo, hi


def moe_combine_exact(down_bits: np.ndarray, rows_of: np.ndarray, weight: np.ndarray) -> np.ndarray:
    """sum_j weight[t][j] * down[rows_of[t][j]] in fp64 ``[T][H]``."""
    down = o.bf16_to_f64(down_bits)
    rows = down.shape[0]
    T, k = rows_of.shape
    out = np.zeros((T, down.shape[1]), dtype=np.float64)
    for j in range(k):
        r = rows_of[:, j].astype(np.int64)
        ok = (r >= 0) & (r < rows)
        out[ok] += np.float64(1.0) * weight[ok, j].astype(np.float64)[:, None] * down[r[ok]]
    return out


def moe_combine(down_bits, rows_of, weight) -> np.ndarray:
    """bf16 bits of the combine."""
    return o.bf16_rne(moe_combine_exact(down_bits, rows_of, weight))


def combine_tolerance(down_bits, rows_of, weight, ref_bits) -> np.ndarray:
    """Per element: 1 bf16 ulp of the reference plus the fp32 summation bound
    2 * (top_k + 1) * 2**-24 * sum_j |weight * down| (the kernel adds the
    terms in fp32, one rounding per product and per sum)."""
    down = np.abs(o.bf16_to_f64(down_bits))
    rows = down.shape[0]
    T, k = rows_of.shape
    mag = np.zeros((T, down.shape[1]), dtype=np.float64)
    for j in range(k):
        r = rows_of[:, j].astype(np.int64)
        ok = (r >= 0) & (r < rows)
        mag[ok] += np.abs(weight[ok, j].astype(np.float64))[:, None] * down[r[ok]]
    return o.bf16_ulp(ref_bits) + 2.0 * (k + 1) * 2.0 ** -24 * mag


def expert_of_rows(offsets: np.ndarray, rows: int) -> np.ndarray:
    """Expert of each row (-1 for rows outside every range)."""
    e = np.full(rows, -1, dtype=np.int64)
    for i in range(len(offsets) - 1):
        e[int(offsets[i]):int(offsets[i + 1])] = i
    return e


def moe_ffn(x_bits, gs_x, row_token, offsets, w_gu, w_gu_sf, alpha_gu, gs_h, w_d, w_d_sf, alpha_d, token_rows,
            token_weight, I: int, tokens=None):
    """One MoE layer's experts (bf16 bits ``[T][H]``, or the rows of
    ``tokens`` only): for every row r of a requested token, with e its expert,
      gu[r]   = bf16(alpha_gu[e] * A[r] . W_gu[e]),  A[r] = NVFP4(x[row_token[r]], gs_x)
      h[r]    = NVFP4(swiglu(gu[r]), gs_h)
      down[r] = bf16(alpha_d[e] * h[r] . W_d[e])
    then the combine of each token's rows.  Rows are independent, so a
    subset of tokens is computed from their own rows alone.
    w_gu: ``[E][2I][H/2]`` codes (unpacked), w_d: ``[E][H][I/2]``."""
    T, H = x_bits.shape
    rows = len(row_token)
    tokens = np.arange(T) if tokens is None else np.asarray(tokens)
    need = np.unique(token_rows[tokens].reshape(-1))
    need = need[(need >= 0) & (need < rows)]
    eor = expert_of_rows(np.asarray(offsets), rows)
    x32 = o.bf16_bits_to_f32(x_bits)
    down = np.zeros((rows, H), dtype=np.uint16)
    for e in np.unique(eor[need]):
        if e < 0:
            continue
        rr = need[eor[need] == e]
        a, a_sf = o.quantize(o.gather_rows(x32, row_token[rr], len(rr)), np.float32(gs_x))
        ag = np.float32(1.0) if alpha_gu is None else np.float32(alpha_gu[e])
        gu = o.gemm(a, a_sf, w_gu[e], w_gu_sf[e], ag)
        hq, hsf = swiglu_quantize(gu, I, gs_h)
        ad = np.float32(1.0) if alpha_d is None else np.float32(alpha_d[e])
        down[rr] = o.gemm(hq, hsf, w_d[e], w_d_sf[e], ad)
    return moe_combine(down, token_rows[tokens], token_weight[tokens]), down
