"""Pins of the oracle's fused-quantisation grouped GEMM (CPU): the bf16 decode
against torch's cast on every pattern, the row gather, a lossless closed form,
and row independence against the single GEMM of each row."""
import numpy as np
import torch

from oracle import nvfp4_ref as o

E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float32)


def _bf16_bits(x32: np.ndarray) -> np.ndarray:
    # truncation is exact for the values used below (they are bf16 values)
    return (np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_bf16_decode_matches_torch_on_all_patterns():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = o.bf16_bits_to_f32(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()
    nan = np.isnan(ref)
    assert (np.isnan(ours) == nan).all()
    np.testing.assert_array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_gather_rows():
    x = np.arange(5 * 32, dtype=np.float32).reshape(5, 32)
    np.testing.assert_array_equal(o.gather_rows(x, None, 3), x[:3])
    got = o.gather_rows(x, [4, 4, 0, -1, 5, 2], 6)
    np.testing.assert_array_equal(got[[0, 1, 2, 5]], x[[4, 4, 0, 2]])
    assert (got[3] == 0).all() and (got[4] == 0).all()


def test_lossless_rows_give_a_plain_matmul():
    # every 16-block holds a +-6 and only e2m1 grid values, gs = 1: the
    # quantiser keeps every value exactly (scale 1, r = 1), so D is the bf16
    # of the exact product of the activations with the dequantised weights
    rng = np.random.default_rng(3)
    T, K, N, E = 6, 64, 5, 2
    x = rng.choice(E2M1_GRID, size=(T, K)) * rng.choice([-1.0, 1.0], size=(T, K)).astype(np.float32)
    x[:, ::16] = 6.0
    x = x.astype(np.float32)
    tok = np.array([5, 0, 3, 3, 1], dtype=np.int32)
    off = np.array([0, 2, 5], dtype=np.int32)
    b = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
    bsf = rng.integers(0x30, 0x40, size=(E, N, K // 16), dtype=np.uint8)
    d = o.grouped_gemm_fused(_bf16_bits(x), tok, np.float32(1.0), b, bsf, off, None,
                             np.zeros((5, N), np.uint16), 5)
    for e in range(E):
        xb = o.dequant(b[e], bsf[e])
        rows = x[tok[off[e]:off[e + 1]]].astype(np.float64)
        np.testing.assert_array_equal(d[off[e]:off[e + 1]], o.bf16_rne(rows @ xb.T))


def test_each_row_is_its_own_quantised_token_times_its_expert():
    rng = np.random.default_rng(11)
    T, K, N, E = 7, 96, 9, 3
    x = (rng.standard_normal((T, K)) * 3).astype(np.float32)
    xb = _bf16_bits(x)
    gs = np.float32(2688.0) / np.float32(np.abs(o.bf16_bits_to_f32(xb)).max())
    tok = np.array([2, 2, 6, -3, 0, 1, 7, 4], dtype=np.int32)  # a repeat, two invalid tokens
    off = np.array([0, 3, 3, 8], dtype=np.int32)               # one empty expert
    b = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
    bsf = rng.integers(0x28, 0x40, size=(E, N, K // 16), dtype=np.uint8)
    alpha = np.array([0.5, 2.0, 0.25], dtype=np.float32)
    init = np.full((9, N), 0x7FC1, np.uint16)
    d = o.grouped_gemm_fused(xb, tok, gs, b, bsf, off, alpha, init, 8)
    x32 = o.bf16_bits_to_f32(xb)
    for e in range(E):
        for i in range(off[e], off[e + 1]):
            row = x32[tok[i]:tok[i] + 1] if 0 <= tok[i] < T else np.zeros((1, K), np.float32)
            qa, sfa = o.quantize(row, gs)
            np.testing.assert_array_equal(d[i], o.gemm(qa, sfa, b[e], bsf[e], alpha[e])[0])
    assert (d[8] == 0x7FC1).all()
    # quantising before or after the gather is the same with one encode scale
    qa_all, sfa_all = o.quantize(x32, gs)
    qa_g, sfa_g = o.quantize(o.gather_rows(x32, tok, 8), gs)
    ok = (tok >= 0) & (tok < T)
    np.testing.assert_array_equal(qa_g[ok], qa_all[tok[ok]])
    np.testing.assert_array_equal(sfa_g[ok], sfa_all[tok[ok]])
