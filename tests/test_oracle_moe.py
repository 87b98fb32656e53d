"""Pins of the MoE FFN oracle (CPU): silu against scipy's logistic function
and its odd-part identity, SwiGLU quantisation in a region where h is exact,
the combine on one-hot and invalid rows, and the FFN against a per-token
route through the single GEMM."""
import numpy as np
import scipy.special

from oracle import moe_ref as m
from oracle import nvfp4_ref as o


def _bits(x32):
    return (np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_silu_against_library_and_identity():
    g = np.linspace(-60, 60, 20001)
    np.testing.assert_allclose(m.silu(g), g * scipy.special.expit(g), rtol=1e-14, atol=1e-300)
    # silu(g) - silu(-g) = g (sigma(g) + sigma(-g) = 1)
    np.testing.assert_allclose(m.silu(g) - m.silu(-g), g, rtol=1e-13, atol=1e-13)
    assert m.silu(0.0) == 0.0 and m.silu(-1000.0) == 0.0 and not np.isnan(m.silu(-1000.0))
    assert m.silu(60.0) == 60.0


def test_swiglu_quantize_where_h_is_exact():
    # gate = 40: silu(40) = 40 (1 - 4e-18), so h = 40 * up exactly in fp32
    # (40 * a bf16 value needs at most 11 significant bits)
    rng = np.random.default_rng(2)
    rows, I = 5, 64
    up = rng.standard_normal((rows, I)).astype(np.float32)
    up = o.bf16_bits_to_f32(_bits(up))
    gu = np.concatenate([np.full((rows, I), 40.0, np.float32), up], axis=1)
    q, sf = m.swiglu_quantize(_bits(gu), I, np.float32(0.7))
    rq, rsf = o.quantize((np.float32(40.0) * up).astype(np.float32), np.float32(0.7))
    np.testing.assert_array_equal(q, rq)
    np.testing.assert_array_equal(sf, rsf)
    # gate = -80: silu underflows to -0, every code is a signed zero
    gu[:, :I] = -80.0
    q, sf = m.swiglu_quantize(_bits(gu), I)
    assert (sf == 0).all() and ((q & 0x77) == 0).all()


def test_combine_one_hot_and_invalid_rows():
    rng = np.random.default_rng(4)
    rows, H, T, k = 10, 24, 4, 3
    down = _bits(rng.standard_normal((rows, H)).astype(np.float32))
    rows_of = np.array([[3, -1, 12], [0, 1, 2], [9, 9, 9], [5, 6, 7]], dtype=np.int32)
    w = np.array([[1.0, 5.0, 7.0], [0.5, 0.25, 0.25], [1.0, 1.0, -1.0], [0.0, 0.0, 0.0]], dtype=np.float32)
    out = m.moe_combine(down, rows_of, w)
    np.testing.assert_array_equal(out[0], down[3])                  # invalid rows add nothing
    np.testing.assert_array_equal(out[2], down[9])                  # 1 + 1 - 1
    assert (o.bf16_to_f64(out[3]) == 0).all()
    exact = 0.5 * o.bf16_to_f64(down[0]) + 0.25 * o.bf16_to_f64(down[1]) + 0.25 * o.bf16_to_f64(down[2])
    np.testing.assert_array_equal(out[1], o.bf16_rne(exact))
    # the order of a token's rows does not change the exact sum
    np.testing.assert_array_equal(m.moe_combine(down, rows_of[:, ::-1], w[:, ::-1]), out)


def test_ffn_equals_a_per_token_route():
    rng = np.random.default_rng(9)
    T, H, I, E, k = 6, 64, 32, 3, 2
    x = _bits((rng.standard_normal((T, H)) * 2).astype(np.float32))
    # token t goes to experts (t % E, (t + 1) % E); rows sorted by expert
    pairs = sorted((e, t, j) for t in range(T) for j, e in enumerate([t % E, (t + 1) % E]))
    row_token = np.array([t for _, t, _ in pairs], dtype=np.int32)
    offsets = np.searchsorted([e for e, _, _ in pairs], np.arange(E + 1)).astype(np.int32)
    token_rows = np.zeros((T, k), dtype=np.int32)
    for r, (_, t, j) in enumerate(pairs):
        token_rows[t, j] = r
    tw = rng.uniform(0.1, 1.0, (T, k)).astype(np.float32)
    w_gu = rng.integers(0, 256, (E, 2 * I, H // 2), dtype=np.uint8)
    w_gu_sf = rng.integers(0x30, 0x3C, (E, 2 * I, H // 16), dtype=np.uint8)
    w_d = rng.integers(0, 256, (E, H, I // 2), dtype=np.uint8)
    w_d_sf = rng.integers(0x30, 0x3C, (E, H, I // 16), dtype=np.uint8)
    a_gu = np.array([0.5, 1.0, 2.0], np.float32)
    a_d = np.array([0.25, 0.5, 1.0], np.float32)
    gs_x, gs_h = np.float32(300.0), np.float32(0.05)
    out, _ = m.moe_ffn(x, gs_x, row_token, offsets, w_gu, w_gu_sf, a_gu, gs_h, w_d, w_d_sf, a_d, token_rows, tw, I)
    x32 = o.bf16_bits_to_f32(x)
    for t in range(T):
        acc = np.zeros(H)
        for j, e in enumerate([t % E, (t + 1) % E]):
            qa, sfa = o.quantize(x32[t:t + 1], gs_x)
            gu = o.gemm(qa, sfa, w_gu[e], w_gu_sf[e], a_gu[e])
            g, u = o.bf16_to_f64(gu[:, :I]), o.bf16_to_f64(gu[:, I:])
            h = (g / (1.0 + np.exp(-g)) * u).astype(np.float32)
            hq, hsf = o.quantize(h, gs_h)
            acc += np.float64(tw[t, j]) * o.bf16_to_f64(o.gemm(hq, hsf, w_d[e], w_d_sf[e], a_d[e]))[0]
        np.testing.assert_array_equal(out[t], o.bf16_rne(acc))
    # a subset of tokens gives the same rows
    sub, _ = m.moe_ffn(x, gs_x, row_token, offsets, w_gu, w_gu_sf, a_gu, gs_h, w_d, w_d_sf, a_d, token_rows, tw, I,
                       tokens=[4, 1])
    np.testing.assert_array_equal(sub, out[[4, 1]])
