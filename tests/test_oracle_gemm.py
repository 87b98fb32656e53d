"""Pins for the oracle's GEMM, grouped GEMM and tolerance (CPU only).

The pins: a hand-worked fixture; closed forms that reduce to an integer
matmul; one-hot operands; exact invariants (sign flip, power-of-two alpha,
permutations, scale exponent shifts) checked through the exact int64 mode;
and a brute-force rational evaluation on tiny shapes.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import synth
from oracle import nvfp4_ref as o

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rows(hexes, per):
    return np.frombuffer(b"".join(bytes.fromhex(h) for h in hexes), np.uint8).reshape(-1, per).copy()


def _worked():
    with open(os.path.join(GOLD, "worked_gemm_2x3x32.json")) as f:
        g = json.load(f)
    K = g["K"]
    a = _rows(g["a_hex"], K // 2)
    asf = _rows(g["a_sf_hex"], K // 16)
    b = _rows(g["b_hex"], K // 2)
    bsf = _rows(g["b_sf_hex"], K // 16)
    return g, a, asf, b, bsf


def test_worked_fixture():
    g, a, asf, b, bsf = _worked()
    d = o.bf16_to_f64(o.gemm(a, asf, b, bsf, np.float32(g["alpha"])))
    np.testing.assert_array_equal(d, np.array(g["expected"]))
    d = o.bf16_to_f64(o.gemm(a, asf, b, bsf, np.float32(0.5)))
    np.testing.assert_array_equal(d, np.array(g["alpha_half_expected"]))


def _torch_bf16_bits(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_unit_scales_reduce_to_integer_matmul():
    # all scales 1.0 (0x38): D = bf16(half-integer matmul); 2*E2M1 are integers
    rng = np.random.default_rng(1)
    M, N, K = 24, 40, 256
    ca = rng.integers(0, 16, size=(M, K)).astype(np.uint8)
    cb = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    two = np.array([0, 1, 2, 3, 4, 6, 8, 12, 0, -1, -2, -3, -4, -6, -8, -12], np.int64)
    s4 = two[ca] @ two[cb].T                      # = 4 * S exactly
    pack = lambda c: (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)
    sfa = np.full((M, K // 16), 0x38, np.uint8)
    sfb = np.full((N, K // 16), 0x38, np.uint8)
    d = o.gemm(pack(ca), sfa, pack(cb), sfb, np.float32(1))
    np.testing.assert_array_equal(d, _torch_bf16_bits(s4 / 4.0))


def test_one_hot_rows_select_b_values():
    # A row m has code 0x2 (=1.0) at column k_m, scale 1; D[m, n] = bf16(xB[n, k_m])
    rng = np.random.default_rng(2)
    M, N, K = 8, 16, 64
    b = synth.random_codes(21, N, K)
    bsf = synth.random_scale_bytes(22, N, K)
    ks = rng.choice(K, size=M, replace=False)
    ca = np.zeros((M, K), np.uint8)
    ca[np.arange(M), ks] = 0x2
    a = (ca[:, 0::2] | (ca[:, 1::2] << 4)).astype(np.uint8)
    asf = np.full((M, K // 16), 0x38, np.uint8)
    # B values from the golden e2m1 table and torch's e4m3 decode
    with open(os.path.join(GOLD, "e2m1_codes.json")) as f:
        e2 = {int(k): v for k, v in json.load(f)["values"].items()}
    cb = np.empty((N, K), np.uint8)
    cb[:, 0::2] = b & 0xF
    cb[:, 1::2] = b >> 4
    sv = torch.from_numpy(bsf.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    xb = np.vectorize(lambda c: e2[int(c)])(cb) * np.repeat(sv, 16, axis=1)
    want = _torch_bf16_bits(xb[:, ks].T)          # exact in fp32 (<= 6 significant bits)
    # compared as values: a -0 term summed with +0 terms is +0
    np.testing.assert_array_equal(o.bf16_to_f64(o.gemm(a, asf, b, bsf, np.float32(1))), o.bf16_to_f64(want))


def _case(seed, M=16, N=24, K=128):
    a = synth.random_codes(seed, M, K)
    b = synth.random_codes(seed + 1, N, K)
    asf = synth.random_scale_bytes(seed + 2, M, K, lo=0x08, hi=0x76)
    bsf = synth.random_scale_bytes(seed + 3, N, K, lo=0x00, hi=0x7E)
    return a, asf, b, bsf


def test_exact_int_mode_agrees_with_fp64():
    for seed in range(3):
        a, asf, b, bsf = _case(100 * seed, 32, 48, 1024)
        s = o.gemm_fp64(a, asf, b, bsf)
        si = o.gemm_exact_int(a, asf, b, bsf).astype(np.float64) * 2.0 ** -20
        ax = np.abs(o.dequant(a, asf)) @ np.abs(o.dequant(b, bsf)).T
        assert (np.abs(s - si) <= 1024 * 2.0 ** -52 * ax).all()


def test_sign_flip_negates_exactly():
    a, asf, b, bsf = _case(5)
    s = o.gemm_exact_int(a, asf, b, bsf)
    s_neg = o.gemm_exact_int(a ^ np.uint8(0x88), asf, b, bsf)
    np.testing.assert_array_equal(s_neg, -s)
    d = o.bf16_to_f64(o.gemm(a, asf, b, bsf))
    dn = o.bf16_to_f64(o.gemm(a ^ np.uint8(0x88), asf, b, bsf))
    np.testing.assert_array_equal(dn, -d)


def test_power_of_two_alpha_scales_exactly():
    a, asf, b, bsf = _case(6)
    d1 = o.bf16_to_f64(o.gemm(a, asf, b, bsf, np.float32(1)))
    for j in (-3, 1, 5):
        dj = o.bf16_to_f64(o.gemm(a, asf, b, bsf, np.float32(2.0 ** j)))
        np.testing.assert_array_equal(dj, d1 * 2.0 ** j)


def test_row_permutation_and_joint_block_permutation():
    a, asf, b, bsf = _case(7, K=256)
    s = o.gemm_exact_int(a, asf, b, bsf)
    p = np.random.default_rng(0).permutation(a.shape[0])
    np.testing.assert_array_equal(o.gemm_exact_int(a[p], asf[p], b, bsf), s[p])
    # permute the 16-element K blocks of A and B together: S unchanged
    nb = a.shape[1] // 8
    bp = np.random.default_rng(1).permutation(nb)
    perm_bytes = lambda x: x.reshape(x.shape[0], nb, 8)[:, bp].reshape(x.shape)
    s2 = o.gemm_exact_int(perm_bytes(a), asf[:, bp], perm_bytes(b), bsf[:, bp])
    np.testing.assert_array_equal(s2, s)


def test_scale_exponent_step_doubles_one_block():
    a, asf, b, bsf = _case(8, K=256)
    s = o.gemm_exact_int(a, asf, b, bsf)
    asf2 = asf.copy()
    asf2[:, 3] += 8                               # e4m3 exponent + 1 (normal codes only)
    s2 = o.gemm_exact_int(a, asf2, b, bsf)
    # contribution of block 3 alone
    mask = np.zeros(a.shape[1], bool)
    mask[3 * 8:4 * 8] = True
    a3 = np.where(mask, a, 0).astype(np.uint8)
    c3 = o.gemm_exact_int(a3, asf, b, bsf)
    np.testing.assert_array_equal(s2 - s, c3)


def _frac_e2m1(c):
    sign = -1 if c & 8 else 1
    e, m = (c >> 1) & 3, c & 1
    return sign * (Fraction(m, 2) if e == 0 else Fraction(2) ** (e - 1) * (1 + Fraction(m, 2)))


def _frac_e4m3(b):
    sign = -1 if b & 0x80 else 1
    e, m = (b >> 3) & 15, b & 7
    return sign * (Fraction(m, 512) if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7))


def _frac_bf16(x: Fraction) -> float:
    """exact RNE of a rational to bf16 (8 significant bits), value as float"""
    if x == 0:
        return 0.0
    sign = -1 if x < 0 else 1
    x = abs(x)
    e = x.numerator.bit_length() - x.denominator.bit_length()
    while Fraction(2) ** e > x:
        e -= 1
    while Fraction(2) ** (e + 1) <= x:
        e += 1
    q = x / Fraction(2) ** (e - 7)                # in [128, 256)
    fl = q.numerator // q.denominator
    rem = q - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * float(Fraction(fl) * Fraction(2) ** (e - 7))


@pytest.mark.parametrize("seed", [0, 1])
def test_brute_force_rational_tiny(seed):
    M, N, K = 5, 7, 48
    a = synth.random_codes(300 + seed, M, K)
    b = synth.random_codes(310 + seed, N, K)
    asf = synth.random_scale_bytes(320 + seed, M, K, signed=True)
    bsf = synth.random_scale_bytes(330 + seed, N, K, signed=True)
    alpha = np.float32(0.3)
    d = o.bf16_to_f64(o.gemm(a, asf, b, bsf, alpha))
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                ca = (int(a[m, k // 2]) >> (4 * (k % 2))) & 0xF
                cb = (int(b[n, k // 2]) >> (4 * (k % 2))) & 0xF
                acc += _frac_e2m1(ca) * _frac_e4m3(int(asf[m, k // 16])) * _frac_e2m1(cb) * _frac_e4m3(int(bsf[n, k // 16]))
            assert d[m, n] == _frac_bf16(acc * Fraction(float(alpha))), (m, n)


def test_grouped_equals_per_expert_and_keeps_untouched_rows():
    E, N, K = 6, 32, 64
    offsets = np.array([0, 3, 3, 10, 11, 11, 20], np.int32)
    rows = 24                                   # rows 20..23 belong to no expert
    a = synth.random_codes(40, rows, K)
    asf = synth.random_scale_bytes(41, rows, K)
    b = np.stack([synth.random_codes(50 + e, N, K) for e in range(E)])
    bsf = np.stack([synth.random_scale_bytes(60 + e, N, K) for e in range(E)])
    alpha = np.array([1, 0.5, 2, 0.25, 1, 4], np.float32)
    sentinel = np.full((rows, N), 0x7FC1, np.uint16)
    d = o.grouped_gemm(a, asf, b, bsf, offsets, alpha, sentinel)
    for e in range(E):
        lo, hi = offsets[e], offsets[e + 1]
        if hi > lo:
            np.testing.assert_array_equal(d[lo:hi], o.gemm(a[lo:hi], asf[lo:hi], b[e], bsf[e], alpha[e]))
    assert (d[20:] == 0x7FC1).all()


def test_tolerance_accepts_fp32_sums_and_rejects_planted_mistakes():
    xa32 = synth.normal_f32(90, (32, 2048))
    xb32 = synth.normal_f32(91, (64, 2048), 0.02)
    gsa, gsb = o.global_encode_scale(xa32), o.global_encode_scale(xb32)
    a, asf = o.quantize(xa32, gsa)
    b, bsf = o.quantize(xb32, gsb)
    alpha = o.alpha_from_scales(gsa, gsb)
    ref = o.gemm(a, asf, b, bsf, alpha)
    tol = o.gemm_tolerance(a, asf, b, bsf, alpha, ref)
    xa, xb = o.dequant(a, asf).astype(np.float32), o.dequant(b, bsf).astype(np.float32)
    # a sequential fp32 accumulation (worst plain order) stays inside the bound
    acc = np.zeros((32, 64), np.float32)
    for k in range(xa.shape[1]):
        acc += np.outer(xa[:, k], xb[:, k]).astype(np.float32)
    d32 = o.bf16_rne((acc * alpha).astype(np.float64))
    err = np.abs(o.bf16_to_f64(d32) - o.bf16_to_f64(ref))
    assert (err <= tol).all()
    # planted mistakes: one K block dropped, or alpha off by 2 %
    a_drop = a.copy()
    a_drop[:, 8:16] = 0
    bad = o.gemm(a_drop, asf, b, bsf, alpha)
    assert (np.abs(o.bf16_to_f64(bad) - o.bf16_to_f64(ref)) > tol).mean() > 0.5
    bad2 = o.gemm(a, asf, b, bsf, alpha * np.float32(1.02))
    assert (np.abs(o.bf16_to_f64(bad2) - o.bf16_to_f64(ref)) > tol).mean() > 0.5


def test_routing_workload_shape():
    tok, off = synth.routing(synth.GROUPED["seed_router"], 512, 256, 8)
    assert off[0] == 0 and off[-1] == 4096 and (np.diff(off) >= 0).all()
    counts = np.bincount(tok, minlength=512)
    assert (counts == 8).all()
    for e in range(256):
        t = tok[off[e]:off[e + 1]]
        assert (np.diff(t) > 0).all()            # token order inside an expert, no repeats
