"""Oracle evaluations of the full-size workloads, spread over a pool of CPU
processes (test infrastructure: numpy, the oracle and the seeded input
generators only; nothing here touches the GPU or the HIP library).

The full-output parity tests compare every element of the largest outputs
(16384 x 6144 GEMMs, 256 experts) with the oracle.  The oracle is plain
numpy and single-threaded outside BLAS, so row blocks and experts are handed
to worker processes; each worker evaluates the oracle functions on its share
exactly as a single call would (rows of a GEMM are independent), and returns
either the oracle's bytes or the comparison counts of its share.
"""
from __future__ import annotations

import math
import multiprocessing as mp
import os

import numpy as np

import synth
from oracle import moe_ref as m
from oracle import mxfp4_ref as mx
from oracle import nvfp4_ref as o


def workers() -> int:
    """Worker processes: the CPUs this process may use, at most 15 (a GPU
    box gives one GPU's job 16 CPUs; one stays with the test process)."""
    return max(1, min(15, len(os.sched_getaffinity(0)) - 1))


def make_pool(n: int | None = None):
    """A spawn-context pool (children start clean: no GPU state, one BLAS
    thread each)."""
    keep = {k: os.environ.get(k) for k in ("OPENBLAS_NUM_THREADS", "OMP_NUM_THREADS")}
    os.environ["OPENBLAS_NUM_THREADS"] = "1"
    os.environ["OMP_NUM_THREADS"] = "1"
    try:
        return mp.get_context("spawn").Pool(n or workers())
    finally:
        for k, v in keep.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


# ---------------------------------------------------------------------------
# Quantisation of row blocks.
# ---------------------------------------------------------------------------
def quantize_block(args):
    x, gs = args
    return o.quantize(x, np.float32(gs))


# ---------------------------------------------------------------------------
# The exhaustive e2m1 rounding sweep.
# ---------------------------------------------------------------------------
def e2m1_codes_of_patterns(args):
    """The oracle's e2m1 codes of the fp32 values of bit patterns [lo, hi)
    (sign bit set when negative)."""
    lo, hi, negative = args
    return o.e2m1_encode(synth.fp32_bit_patterns(lo, hi, negative))


# ---------------------------------------------------------------------------
# Element-by-element comparison of GPU output rows with the oracle.
# ---------------------------------------------------------------------------
class Stats:
    """Counts of one comparison, summed over blocks: elements, elements
    outside the per-element bound, worst excess over it, the squared error
    and squared norm for the relative Frobenius error, and elements within
    2 bf16 ulps."""

    def __init__(self):
        self.n = self.bad = self.strict = 0
        self.excess = -math.inf
        self.err2 = self.ref2 = 0.0
        self.nan_mismatch = 0

    def add(self, other: "Stats"):
        self.n += other.n
        self.bad += other.bad
        self.strict += other.strict
        self.excess = max(self.excess, other.excess)
        self.err2 += other.err2
        self.ref2 += other.ref2
        self.nan_mismatch += other.nan_mismatch
        return self

    @property
    def frob(self) -> float:
        return math.sqrt(self.err2 / self.ref2) if self.ref2 > 0 else math.sqrt(self.err2)

    def check(self, label: str, strict_frac: float | None = 0.999):
        assert self.nan_mismatch == 0, f"{label}: NaN pattern differs in {self.nan_mismatch} elements"
        assert self.bad == 0, (f"{label}: {self.bad} of {self.n} elements outside tolerance; "
                               f"worst excess {self.excess:.3g}")
        assert self.frob <= 1e-2, f"{label}: relative Frobenius error {self.frob}"
        if strict_frac is not None and self.n:
            assert self.strict / self.n > strict_frac, f"{label}: {self.strict} of {self.n} within 2 bf16 ulps"
        return self


def compare(d_bits: np.ndarray, s: np.ndarray, tol: np.ndarray, ref_bits: np.ndarray) -> Stats:
    """Stats of GPU bf16 bits against the oracle's exact sum s (already times
    alpha), its bf16 rounding ref_bits and the per-element bound tol."""
    st = Stats()
    got, want = o.bf16_to_f64(d_bits), o.bf16_to_f64(ref_bits)
    nan_g, nan_w = np.isnan(got), np.isnan(want)
    st.nan_mismatch = int((nan_g != nan_w).sum())
    ok = ~nan_w
    err = np.abs(got[ok] - want[ok])
    t = tol[ok]
    st.n = int(err.size)
    st.bad = int((err > t).sum())
    if err.size:
        st.excess = float(np.max(err - t))
    st.err2 = float(np.sum((got[ok] - s[ok]) ** 2))
    st.ref2 = float(np.sum(s[ok] ** 2))
    st.strict = int((err <= 2 * o.bf16_ulp(ref_bits)[ok]).sum())
    return st


def _oracle_rows(xa, xb, alpha):
    """(exact sum times alpha, its bf16 bits, per-element bound) for
    dequantised rows xa against xb."""
    s = (xa @ xb.T) * np.float64(np.float32(alpha))
    ref = o.bf16_rne(s)
    return s, ref, o.tolerance_dequantized(xa, xb, alpha, ref)


def gemm_rows_compare(args):
    """Rows [r0, r1) of an NVFP4 (fmt 'nv') or MXFP4 (fmt 'mx') GEMM: the
    oracle on those rows, compared with each GPU output given for them."""
    fmt, qa, sfa, qb, sfb, alpha, outs = args
    deq = o.dequant if fmt == "nv" else mx.dequant
    s, ref, tol = _oracle_rows(deq(qa, sfa), deq(qb, sfb), alpha)
    return [compare(d, s, tol, ref) for d in outs]


# ---------------------------------------------------------------------------
# The grouped MoE workload: 256 experts of N(0, 0.02) weights quantised one
# expert at a time with the expert's own encode scale.
# ---------------------------------------------------------------------------
def expert_oracle(args):
    """Expert e: its weights, their encode scale and NVFP4 bytes, alpha =
    1 / (gs_a * gs_e), and the oracle's output rows for each activation set
    given (A codes and scales of the expert's rows)."""
    e, gs_a, a_sets, n, k = args
    w = synth.expert_weights(e, n, k)
    gs = o.global_encode_scale(w)
    qb, sfb = o.quantize(w, gs)
    alpha = o.alpha_from_scales(gs_a, gs)
    xb = o.dequant(qb, sfb)
    rows = [_oracle_rows(o.dequant(qa, sfa), xb, alpha) for qa, sfa in a_sets]
    return e, qb, sfb, np.float32(gs), np.float32(alpha), rows


# ---------------------------------------------------------------------------
# The MoE expert FFN at the pages' shape, one expert at a time.
# ---------------------------------------------------------------------------
def ffn_expert_weights(seed: int, e: int, H: int, I: int):
    """Expert e's seeded random gate/up ([2I][H/2], [2I][H/16]) and down
    ([H][I/2], [H][I/16]) codes and scale bytes."""
    base = seed + 10 * e
    w_gu = synth.random_codes(base + 2, 2 * I, H)
    w_gu_sf = synth.random_scale_bytes(base + 3, 2 * I, H, lo=0x28, hi=0x38)
    w_d = synth.random_codes(base + 4, H, I)
    w_d_sf = synth.random_scale_bytes(base + 5, H, I, lo=0x28, hi=0x38)
    return w_gu, w_gu_sf, w_d, w_d_sf


def ffn_expert_oracle(args):
    """Expert e of the FFN, three checks on its rows:
    * the gate/up GEMM on the oracle-quantised activations (exact sum, bits,
      bound), compared with the GPU's gate/up output gu_gpu;
    * the down GEMM fed with the GPU's own h codes and scales (hq, hsf),
      compared with the GPU's down output down_gpu;
    * the pure-oracle chain (oracle gate/up -> SwiGLU -> quantise -> down)
      as bf16 bits, for the layer's end-to-end comparison."""
    seed, e, H, I, qa, sfa, a_gu, gs_h, a_d, gu_gpu, hq, hsf, down_gpu = args
    w_gu, w_gu_sf, w_d, w_d_sf = ffn_expert_weights(seed, e, H, I)
    x_gu, x_d = o.dequant(w_gu, w_gu_sf), o.dequant(w_d, w_d_sf)
    s_gu, ref_gu, tol_gu = _oracle_rows(o.dequant(qa, sfa), x_gu, a_gu)
    st_gu = compare(gu_gpu, s_gu, tol_gu, ref_gu)
    s_d, ref_d, tol_d = _oracle_rows(o.dequant(hq, hsf), x_d, a_d)
    st_d = compare(down_gpu, s_d, tol_d, ref_d)
    cq, csf = m.swiglu_quantize(ref_gu, I, gs_h)
    chain = o.gemm(cq, csf, w_d, w_d_sf, a_d)
    return e, st_gu, st_d, chain
