"""GPU parity of the grouped GEMM that quantises its bf16 activations on load
(nvfp4_grouped_gemm_fused / nvfp4_grouped_gemm_packed_fused), through the C ABI:
against the oracle at the GEMM tolerance, and bit for bit against the unfused
path (the quantise kernel, a row gather and the grouped GEMM on the GPU)."""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_07_amd as nv
import synth
from oracle import nvfp4_ref as o
from tests.gpu_util import bits, check_gemm, dev, gpu_quantize, host, say, scalar

pytestmark = pytest.mark.gpu
SENTINEL = 0x7FC1


def _bf16(x32: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of fp32 values, round to nearest even (torch's cast)."""
    return torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _plan(gk):
    """Grouped kernel 2 (32-row passes) or 3 (64-row passes) for the calls in
    the block; None keeps the library's choice."""
    return nv.forced_plan(nv.FAMILY_GROUPED, -1 if gk is None else gk)


def _fused(x_t, tok_t, gs_t, b_t, bsf_t, off_t, alpha_t, rows, T, N, K, E, packed):
    d = torch.full((max(rows, 1), max(N, 1)), SENTINEL, dtype=torch.int16, device="cuda")
    st = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    fn = nv.nvfp4_grouped_gemm_packed_fused if packed else nv.nvfp4_grouped_gemm_fused
    fn(x_t, tok_t, gs_t, b_t, bsf_t, off_t, alpha_t, d, rows, T, N, K, E, st)
    return d, st


def _unfused(x32_t, tok, gs_t, b_t, bsf_t, off_t, alpha_t, rows, N, K, E, packed):
    """Quantise kernel on the fp32 copy, row gather (zero rows for invalid
    tokens), then the grouped GEMM."""
    q_t, sf_t = gpu_quantize(x32_t, gs_t)
    T = x32_t.shape[0]
    q_t = torch.cat([q_t, torch.zeros_like(q_t[:1])])
    sf_t = torch.cat([sf_t, torch.zeros_like(sf_t[:1])])
    idx = np.where((tok >= 0) & (tok < T), tok, T).astype(np.int64)
    idx_t = torch.from_numpy(idx).cuda()
    qa_t, sfa_t = q_t[idx_t].contiguous(), sf_t[idx_t].contiguous()
    d = torch.full((max(rows, 1), max(N, 1)), SENTINEL, dtype=torch.int16, device="cuda")
    if packed:
        nv.nvfp4_grouped_gemm_packed(qa_t, sfa_t, b_t, bsf_t, off_t, alpha_t, d, rows, N, K, E)
    else:
        nv.nvfp4_grouped_gemm(qa_t, sfa_t, b_t, bsf_t, off_t, alpha_t, d, rows, N, K, E, None)
    return d


def _problem(seed=0, T=100, E=6, N=300, K=1024, counts=(0, 1, 33, 70, 17, 64)):
    rng = np.random.default_rng(seed)
    x32 = (rng.standard_normal((T, K)) * 2.0).astype(np.float32)
    x32[3, :16] = 0.0                                  # an all-zero block
    x32[5, 16:32] *= 1e-30                             # a block whose scale underflows to 0
    xb = _bf16(x32)
    xq = o.bf16_bits_to_f32(xb)                        # the values the kernel sees
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    rows = int(off[-1])
    tok = rng.integers(0, T, rows).astype(np.int32)
    tok[2] = tok[1]                                    # a repeated token
    b = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
    bsf = rng.integers(0x28, 0x40, size=(E, N, K // 16), dtype=np.uint8)
    alpha = np.linspace(0.5, 2.0, E).astype(np.float32)
    gs = np.float32(2688.0) / np.float32(np.abs(xq).max())
    return xb, xq, tok, off, rows, b, bsf, alpha, gs


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("gk", [2, 3])
def test_fused_ragged_against_oracle_and_unfused(packed, gk):
    xb, xq, tok, off, rows, b, bsf, alpha, gs = _problem()
    T, K = xq.shape
    E, N = b.shape[:2]
    tok = tok.copy()
    tok[40] = T + 5                                    # an invalid token: zero row, status -(1 + 40)
    say("fused ragged", "packed" if packed else "plain", "gplan", gk, "rows", rows)
    b_t, bsf_t = dev(b), dev(bsf)
    if packed:
        b_t, bsf_t = nv.grouped_pack(b_t, bsf_t, N, K, E)
    x_t = dev(xb.view(np.int16))
    gs_t, off_t, alpha_t, tok_t = scalar(gs), dev(off), dev(alpha), dev(tok)
    with _plan(gk):
        d, st = _fused(x_t, tok_t, gs_t, b_t, bsf_t, off_t, alpha_t, rows, T, N, K, E, packed)
        du = _unfused(dev(xq), tok, gs_t, b_t, bsf_t, off_t, alpha_t, rows, N, K, E, packed)
    assert int(host(st)[0]) == -(1 + 40)
    got = bits(d)
    np.testing.assert_array_equal(got, bits(du))
    qa, sfa = o.quantize(o.gather_rows(xq, tok, rows), gs)
    for e in range(E):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi > lo:
            check_gemm(got[lo:hi], qa[lo:hi], sfa[lo:hi], b[e], bsf[e], alpha[e], f"expert {e}")
    ref = o.grouped_gemm_fused(xb, tok, gs, b, bsf, off, alpha, np.full((rows, N), SENTINEL, np.uint16), rows)
    assert (got[40] == ref[40]).all() and (ref[40] == 0).all()


def test_fused_identity_rows_and_null_scale():
    xb, xq, _, off, rows, b, bsf, alpha, _ = _problem(seed=4, T=200, counts=(10, 0, 40, 66, 5, 79))
    T, K = xq.shape
    E, N = b.shape[:2]
    say("fused identity rows", rows)
    d, st = _fused(dev(xb.view(np.int16)), None, None, dev(b), dev(bsf), dev(off), None, rows, T, N, K, E, False)
    assert int(host(st)[0]) == 0
    got = bits(d)
    qa, sfa = o.quantize(xq[:rows], np.float32(1.0))
    for e in range(E):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi > lo:
            check_gemm(got[lo:hi], qa[lo:hi], sfa[lo:hi], b[e], bsf[e], None, f"expert {e}")


def test_quantize_rows_bf16_bitwise():
    xb, xq, tok, off, rows, b, bsf, alpha, gs = _problem(seed=8)
    T, K = xq.shape
    tok = tok.copy()
    tok[7] = -2
    tok[9] = T
    say("quantize rows bf16", rows, T, K)
    q = torch.empty((rows, K // 2), dtype=torch.uint8, device="cuda")
    sf = torch.empty((rows, K // 16), dtype=torch.uint8, device="cuda")
    nv.nvfp4_quantize_rows_bf16(dev(xb.view(np.int16)), dev(tok), scalar(gs), q, sf, rows, T, K)
    rq, rsf = o.quantize(o.gather_rows(xq, tok, rows), gs)
    np.testing.assert_array_equal(host(q), rq)
    np.testing.assert_array_equal(host(sf), rsf)
    # identity rows, NULL scale
    nv.nvfp4_quantize_rows_bf16(dev(xb.view(np.int16)), None, None, q[:T], sf[:T], T, T, K)
    rq, rsf = o.quantize(xq, np.float32(1.0))
    np.testing.assert_array_equal(host(q)[:T], rq)
    np.testing.assert_array_equal(host(sf)[:T], rsf)


def test_fused_degenerate_calls_report_status():
    # no rows: only the offsets are checked (status 0, nothing written); an
    # invalid range reports its expert; no experts: nothing to do
    K, N, T = 512, 256, 4
    x = torch.zeros((T, K), dtype=torch.int16, device="cuda")
    b = torch.zeros((2, N, K // 2), dtype=torch.uint8, device="cuda")
    bsf = torch.zeros((2, N, K // 16), dtype=torch.uint8, device="cuda")
    d = torch.full((3, N), SENTINEL, dtype=torch.int16, device="cuda")  # 3 rows: the second call writes them
    st = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    say("fused degenerate")
    nv.nvfp4_grouped_gemm_fused(x, None, None, b, bsf, dev(np.array([0, 0, 0], np.int32)), None, d, 0, T, N, K, 2, st)
    assert int(host(st)[0]) == 0 and (bits(d) == SENTINEL).all()
    nv.nvfp4_grouped_gemm_fused(x, None, None, b, bsf, dev(np.array([0, 3, 2], np.int32)), None, d, 3, T, N, K, 2, st)
    assert int(host(st)[0]) == 2
    assert (bits(d) == 0).all()  # expert 0's rows of zero activations; expert 1 skipped
    nv.nvfp4_grouped_gemm_fused(x, None, None, b, bsf, None, None, d, 3, T, N, K, 0, None)
    torch.cuda.synchronize()


def test_grouped_paths_at_maximum_k():
    # K = 2^22 on the plain, packed and fused-packed grouped kernels: 2 experts
    # of 20 rows (one 256-row slab each, mostly padding), 3 + 5 routed rows
    E, N, K, T = 2, 20, 1 << 22, 6
    rng = np.random.default_rng(141)
    x32 = rng.standard_normal((T, K)).astype(np.float32)
    xb = _bf16(x32)
    xq = o.bf16_bits_to_f32(xb)
    gs = o.global_encode_scale(xq)
    tok = np.array([5, 0, 2, 2, 1, 4, 3, 0], dtype=np.int32)
    off = np.array([0, 3, 8], dtype=np.int32)
    rows = 8
    b = synth.random_codes(142, E * N, K).reshape(E, N, K // 2)
    bsf = synth.random_scale_bytes(143, E * N, K, lo=0x30, hi=0x40).reshape(E, N, K // 16)
    alpha = np.array([2.0 ** -10, 2.0 ** -9], np.float32)
    qa, sfa = o.quantize(o.gather_rows(xq, tok, rows), gs)
    b_t, bsf_t, off_t, alpha_t = dev(b), dev(bsf), dev(off), dev(alpha)
    say("max K grouped: plain")
    d = torch.full((rows, N), SENTINEL, dtype=torch.int16, device="cuda")
    nv.nvfp4_grouped_gemm(dev(qa), dev(sfa), b_t, bsf_t, off_t, alpha_t, d, rows, N, K, E, None)
    got_plain = bits(d)
    say("max K grouped: packed and fused")
    pb, psf = nv.grouped_pack(b_t, bsf_t, N, K, E)
    del b_t, bsf_t
    d2 = torch.full((rows, N), SENTINEL, dtype=torch.int16, device="cuda")
    nv.nvfp4_grouped_gemm_packed(dev(qa), dev(sfa), pb, psf, off_t, alpha_t, d2, rows, N, K, E)
    d3, st = _fused(dev(xb.view(np.int16)), dev(tok), scalar(gs), pb, psf, off_t, alpha_t, rows, T, N, K, E, True)
    assert int(host(st)[0]) == 0
    np.testing.assert_array_equal(bits(d2), got_plain)
    np.testing.assert_array_equal(bits(d3), got_plain)
    for e in range(E):
        lo, hi = int(off[e]), int(off[e + 1])
        check_gemm(got_plain[lo:hi], qa[lo:hi], sfa[lo:hi], b[e], bsf[e], alpha[e], f"max K expert {e}")
