"""GPU parity of the MXFP4 GEMM (nvfp4_mx_gemm) with the MX oracle, through
the C ABI: every MX plan (LDS-staged and register tiles) forced on ragged shapes, the attention-projection
sweep with seeded random codes and E8M0 scales, determinism, and the no-op /
error paths that need a device (the large shapes, every element, are in
test_gpu_large.py)."""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_07_amd as nv
import synth
from oracle import mxfp4_ref as mx
from oracle import nvfp4_ref as o
from tests.gpu_util import bits, dev, say, scalar

pytestmark = pytest.mark.gpu

SCALE_LO, SCALE_HI = 120, 134   # E8M0 bytes: 2**-7 .. 2**7, products well inside fp32


def _operands(seed, M, N, K):
    a, b = synth.random_codes(seed, M, K), synth.random_codes(seed + 1, N, K)
    asf = synth.random_scale_bytes(seed + 2, M, 2 * K, SCALE_LO, SCALE_HI)[:, : K // 32].copy()
    bsf = synth.random_scale_bytes(seed + 3, N, 2 * K, SCALE_LO, SCALE_HI)[:, : K // 32].copy()
    return a, asf, b, bsf


def _mx_gemm(a_t, asf_t, b_t, bsf_t, alpha_t, M, N, K, fill=0x7FC1):
    d = torch.full((M, N), fill, dtype=torch.int16, device="cuda")
    ws = nv.mx_gemm_workspace(M, N, K)
    nv.nvfp4_mx_gemm(a_t, asf_t, b_t, bsf_t, alpha_t, d, M, N, K, ws)
    return d


def _check(d_bits, a, asf, b, bsf, alpha, label, rows=None):
    alpha = np.float32(1.0) if alpha is None else np.float32(alpha)
    if rows is not None:
        a, asf, d_bits = a[rows], asf[rows], d_bits[rows]
    s = mx.gemm_fp64(a, asf, b, bsf) * np.float64(alpha)
    ref = o.bf16_rne(s)
    tol = mx.gemm_tolerance(a, asf, b, bsf, alpha, ref)
    got, want = o.bf16_to_f64(d_bits), o.bf16_to_f64(ref)
    assert got.shape == want.shape
    err = np.abs(got - want)
    bad = err > tol
    assert not bad.any(), f"{label}: {bad.sum()} of {bad.size} outside tolerance, worst excess {np.max(err - tol):.3g}"
    den = np.linalg.norm(s)
    frob = np.linalg.norm(got - s) / den if den > 0 else np.linalg.norm(got)
    assert frob <= 1e-2, f"{label}: relative Frobenius error {frob}"
    assert np.mean(err <= 2 * o.bf16_ulp(ref)) > 0.999, label


def test_every_mx_plan_forced_on_ragged_shapes(force_plan):
    # each MX tile, with and without split-K, on shapes that cut every tile edge
    for (M, N, K) in [(200, 330, 1536), (1, 1, 256), (257, 129, 512)]:
        a, asf, b, bsf = _operands(M + N, M, N, K)
        at, asft, bt, bsft = dev(a), dev(asf), dev(b), dev(bsf)
        seen = set()
        for kind in range(10):   # past the last kind the plan falls back to auto
            for splits in (1, 3):
                force_plan(nv.FAMILY_MX, kind, splits)
                plan = nv.nvfp4_mx_gemm_plan(M, N, K)
                if (plan, nv.nvfp4_mx_gemm_workspace_size(M, N, K)) in seen:
                    continue
                seen.add((plan, nv.nvfp4_mx_gemm_workspace_size(M, N, K)))
                say("mx forced", M, N, K, kind, splits, plan)
                d = _mx_gemm(at, asft, bt, bsft, scalar(0.75), M, N, K)
                _check(bits(d), a, asf, b, bsf, np.float32(0.75), f"{M}x{N}x{K} {plan} s{splits}")
                d2 = _mx_gemm(at, asft, bt, bsft, scalar(0.75), M, N, K, fill=0x1234)
                np.testing.assert_array_equal(bits(d2), bits(d), err_msg=f"{plan} rerun not bitwise equal")
        force_plan(nv.FAMILY_MX, -1)


def test_attention_projection_sweep():
    w = synth.WORKLOADS["attn_proj_n768_k6144"]
    N, K = w["n"], w["k"]
    mmax = max(w["ms"])
    a, asf, b, bsf = _operands(7100, mmax, N, K)
    at, asft, bt, bsft = dev(a), dev(asf), dev(b), dev(bsf)
    for m in w["ms"]:
        say("mx sweep", m, N, K, nv.nvfp4_mx_gemm_plan(m, N, K))
        d = _mx_gemm(at[:m], asft[:m], bt, bsft, None, m, N, K)
        _check(bits(d), a[:m], asf[:m], b, bsf, None, f"mx M={m}")


def test_zero_sized_and_bad_k():
    d = torch.zeros((0, 8), dtype=torch.int16, device="cuda")
    x = torch.zeros((16, 128), dtype=torch.uint8, device="cuda")
    nv.nvfp4_mx_gemm(x, x, x, x, None, d, 0, 8, 256)
    with pytest.raises(nv.Nvfp4Error) as e:
        nv.nvfp4_mx_gemm(x, x, x, x, None, d, 4, 8, 48)
    assert e.value.status == 2


def test_every_mx_plan_at_maximum_k(force_plan):
    # K = 2^22 (2 MB code rows, 128 KB scale rows) on every MX plan, with and
    # without split-K, against one oracle evaluation
    M, N, K = 17, 24, 1 << 22
    a, asf, b, bsf = _operands(7300, M, N, K)
    alpha = np.float32(2.0 ** -8)
    say("mx max K oracle")
    s = mx.gemm_fp64(a, asf, b, bsf) * np.float64(alpha)
    ref = o.bf16_rne(s)
    tol = mx.gemm_tolerance(a, asf, b, bsf, alpha, ref)
    want = o.bf16_to_f64(ref)
    at, asft, bt, bsft = dev(a), dev(asf), dev(b), dev(bsf)
    seen = set()
    for kind in range(10):
        for splits in (1, 3):
            force_plan(nv.FAMILY_MX, kind, splits)
            key = (nv.nvfp4_mx_gemm_plan(M, N, K), nv.nvfp4_mx_gemm_workspace_size(M, N, K))
            if key in seen:
                continue
            seen.add(key)
            say("mx max K plan", kind, splits, key)
            got = o.bf16_to_f64(bits(_mx_gemm(at, asft, bt, bsft, scalar(alpha), M, N, K)))
            assert (np.abs(got - want) <= tol).all(), f"{key}: outside tolerance"
            assert np.linalg.norm(got - s) / np.linalg.norm(s) <= 1e-2, key
    force_plan(nv.FAMILY_MX, -1)
    assert len(seen) >= 8
