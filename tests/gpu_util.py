"""Helpers for the GPU parity tests: device copies, calls through the C ABI
binding, and the comparison against the oracle at the tolerance of the
method (bit-exact for bytes; for the bf16 GEMM, relative Frobenius error
<= 1e-2 and the per-element bound of ``oracle.nvfp4_ref.gemm_tolerance``)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import nvfp4_block_scaled_07_amd as nv
from oracle import nvfp4_ref as o

DEV = "cuda"


def say(*msg):
    print("[case]", *msg, flush=True)
    sys.stdout.flush()


def dev(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def scalar(v) -> torch.Tensor:
    return torch.tensor([float(np.float32(v))], dtype=torch.float32, device=DEV)


def gpu_global_scale(x_t: torch.Tensor) -> torch.Tensor:
    gs = torch.empty(1, dtype=torch.float32, device=DEV)
    nv.nvfp4_global_scale(x_t, x_t.numel(), gs)
    return gs


def gpu_quantize(x_t: torch.Tensor, gs_t=None):
    R, K = x_t.shape
    q = torch.empty((R, K // 2), dtype=torch.uint8, device=DEV)
    sf = torch.empty((R, K // 16), dtype=torch.uint8, device=DEV)
    nv.nvfp4_quantize(x_t, R, K, gs_t, q, sf)
    return q, sf


def gpu_gemm(a_t, asf_t, b_t, bsf_t, alpha_t, M, N, K, d_fill=None):
    d = torch.empty((M, N), dtype=torch.int16, device=DEV)
    if d_fill is not None:
        d.fill_(d_fill)
    ws = nv.gemm_workspace(M, N, K)
    nv.nvfp4_gemm(a_t, asf_t, b_t, bsf_t, alpha_t, d, M, N, K, ws)
    return d


def bits(t: torch.Tensor) -> np.ndarray:
    return host(t).view(np.uint16)


def check_gemm(d_bits: np.ndarray, a, asf, b, bsf, alpha, label: str = ""):
    """Compare GPU bf16 bits with the oracle; returns stats."""
    alpha = np.float32(1.0) if alpha is None else np.float32(alpha)
    s = o.gemm_fp64(a, asf, b, bsf) * np.float64(alpha)
    ref = o.bf16_rne(s)
    tol = o.gemm_tolerance(a, asf, b, bsf, alpha, ref)
    got = o.bf16_to_f64(d_bits)
    want = o.bf16_to_f64(ref)
    assert got.shape == want.shape, (got.shape, want.shape)
    nan_g, nan_w = np.isnan(got), np.isnan(want)
    assert (nan_g == nan_w).all(), f"{label}: NaN pattern differs"
    ok = ~nan_w
    err = np.abs(got[ok] - want[ok])
    bad = err > tol[ok]
    assert not bad.any(), (f"{label}: {bad.sum()} of {bad.size} elements outside tolerance; "
                           f"worst excess {np.max(err - tol[ok]):.3g}")
    den = np.linalg.norm(s[ok])
    frob = np.linalg.norm(got[ok] - s[ok]) / den if den > 0 else np.linalg.norm(got[ok])
    assert frob <= 1e-2, f"{label}: relative Frobenius error {frob}"
    strict = np.mean(err <= 2 * o.bf16_ulp(ref)[ok]) if err.size else 1.0
    return dict(frob=float(frob), strict_2ulp_frac=float(strict), n=int(err.size))
