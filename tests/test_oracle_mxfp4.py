"""Pins for the MXFP4 oracle (CPU only).

The pins: torch's own E8M0 decode on all 256 bytes; a hand-worked block;
agreement with the independently pinned NVFP4 oracle wherever the two formats
coincide (power-of-two scales shared by 32 elements); exact Python-integer
evaluation on small shapes; and exact invariants (sign flip, scale exponent
shift, alpha).  A plausible slip in the MX oracle (scale bias, block size,
scale row indexing, operand order) fails at least one of them.
"""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import mxfp4_ref as mx
from oracle import nvfp4_ref as nv


def test_e8m0_decode_matches_torch_on_every_byte():
    b = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = b.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    ours = mx.E8M0_LUT
    assert np.isnan(ours[255]) and np.isnan(ref[255])
    np.testing.assert_array_equal(ours[:255], ref[:255])
    assert ours[127] == 1.0 and ours[128] == 2.0 and ours[0] == 2.0 ** -127 and ours[254] == 2.0 ** 127


def test_hand_worked_block():
    # A: one block of 32 codes 0x2 (1.0) with scale byte 128 (x2);
    # B: 32 codes 0x4 (2.0) with scale byte 126 (x0.5):
    # S = 32 * (1 * 2) * (2 * 0.5) = 64; the second B row flips every sign
    # (0xC = -2.0) and halves nothing else: S = -64.
    a = np.full((1, 16), 0x22, np.uint8)
    asf = np.array([[128]], np.uint8)
    b = np.stack([np.full(16, 0x44, np.uint8), np.full(16, 0xCC, np.uint8)])
    bsf = np.array([[126], [126]], np.uint8)
    s = mx.gemm_fp64(a, asf, b, bsf)
    np.testing.assert_array_equal(s, [[64.0, -64.0]])
    d = nv.bf16_to_f64(mx.gemm(a, asf, b, bsf, np.float32(0.25)))
    np.testing.assert_array_equal(d, [[16.0, -16.0]])


def _pow2_e4m3(byte_e8m0):
    """e4m3fn code of 2**(byte - 127) for exponents in e4m3's normal range."""
    p = byte_e8m0.astype(np.int64) - 127
    assert ((p >= -6) & (p <= 8)).all()
    return ((p + 7) << 3).astype(np.uint8)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_agrees_with_nvfp4_oracle_on_shared_power_of_two_scales(seed):
    # an MX block of 32 with scale 2**p is two NVFP4 blocks of 16 whose e4m3
    # scales are 2**p; the two oracles (separately written and pinned) agree
    M, N, K = 7, 5, 256
    a, b = synth.random_codes(seed, M, K), synth.random_codes(seed + 10, N, K)
    asf = synth.random_scale_bytes(seed + 20, M, 2 * K, 121, 135)[:, : K // 32]
    bsf = synth.random_scale_bytes(seed + 30, N, 2 * K, 121, 135)[:, : K // 32]
    s_mx = mx.gemm_fp64(a, asf, b, bsf)
    s_nv = nv.gemm_fp64(a, np.repeat(_pow2_e4m3(asf), 2, axis=1), b, np.repeat(_pow2_e4m3(bsf), 2, axis=1))
    np.testing.assert_array_equal(s_mx, s_nv)
    # and a block-size slip (scale byte j applied to elements 16 j .. 16 j + 15,
    # the second half of K reusing the first half's bytes) would not agree
    sl = np.tile(np.repeat(mx.E8M0_LUT[asf], 16, axis=1), (1, 2))
    wrong = nv.E2M1_LUT[nv.unpack_codes(a)] * sl
    assert not np.array_equal(wrong @ mx.dequant(b, bsf).T, s_mx)


@pytest.mark.parametrize("seed", [3, 4])
def test_exact_integer_evaluation(seed):
    # scales within [117, 137]: every fp64 partial sum is exact, so the fp64
    # oracle equals the exact integer sum scaled by 2**(2 e_min - 2 - 254)
    M, N, K = 3, 4, 96
    a, b = synth.random_codes(seed, M, K), synth.random_codes(seed + 1, N, K)
    asf = synth.random_scale_bytes(seed + 2, M, 2 * K, 117, 137)[:, : K // 32]
    bsf = synth.random_scale_bytes(seed + 3, N, 2 * K, 117, 137)[:, : K // 32]
    e_min = 117
    exact = mx.gemm_exact_int(a, asf, b, bsf, e_min)
    s = mx.gemm_fp64(a, asf, b, bsf)
    for m in range(M):
        for n in range(N):
            assert s[m, n] == math.ldexp(exact[m][n], 2 * (e_min - 127) - 2)


def test_invariants_sign_scale_shift_alpha():
    M, N, K = 6, 9, 512
    a, b = synth.random_codes(40, M, K), synth.random_codes(41, N, K)
    asf = synth.random_scale_bytes(42, M, 2 * K, 120, 134)[:, : K // 32]
    bsf = synth.random_scale_bytes(43, N, 2 * K, 120, 134)[:, : K // 32]
    s = mx.gemm_fp64(a, asf, b, bsf)
    np.testing.assert_array_equal(mx.gemm_fp64(a ^ 0x88, asf, b, bsf), -s)       # every A sign flipped
    np.testing.assert_array_equal(mx.gemm_fp64(a, asf + 1, b, bsf), 2.0 * s)     # A scales doubled
    bsf2 = bsf.copy()
    bsf2[:, 0] += 3                                                              # one B block x8
    xa, xb = mx.dequant(a, asf), mx.dequant(b, bsf)
    np.testing.assert_array_equal(mx.gemm_fp64(a, asf, b, bsf2), s + 7.0 * (xa[:, :32] @ xb[:, :32].T))
    d1 = nv.bf16_to_f64(mx.gemm(a, asf, b, bsf, np.float32(1.0)))
    d4 = nv.bf16_to_f64(mx.gemm(a, asf, b, bsf, np.float32(4.0)))
    np.testing.assert_array_equal(d4, 4.0 * d1)
    # operand order: D(B, A) is D(A, B) transposed
    np.testing.assert_array_equal(mx.gemm_fp64(b, bsf, a, asf), s.T)


def test_shape_checks_and_nan_scale():
    a = np.zeros((2, 16), np.uint8)
    with pytest.raises(ValueError):
        mx.dequant(a, np.zeros((2, 2), np.uint8))        # K = 32 needs one scale per row
    x = mx.dequant(np.full((1, 16), 0x22, np.uint8), np.array([[255]], np.uint8))
    assert np.isnan(x).all()


def test_tolerance_rejects_planted_mistakes():
    M, N, K = 16, 24, 1024
    a, b = synth.random_codes(50, M, K), synth.random_codes(51, N, K)
    asf = synth.random_scale_bytes(52, M, 2 * K, 122, 132)[:, : K // 32]
    bsf = synth.random_scale_bytes(53, N, 2 * K, 122, 132)[:, : K // 32]
    ref = mx.gemm(a, asf, b, bsf)
    tol = mx.gemm_tolerance(a, asf, b, bsf, np.float32(1), ref)
    refv = nv.bf16_to_f64(ref)
    # a bias of 126 instead of 127 for B (every value doubled)
    bad = nv.bf16_to_f64(mx.gemm(a, asf, b, bsf + 1))
    assert (np.abs(bad - refv) > tol).mean() > 0.9
    # scales of the wrong row (A scale rows rotated by one)
    bad = nv.bf16_to_f64(mx.gemm(a, np.roll(asf, 1, axis=0), b, bsf))
    assert (np.abs(bad - refv) > tol).mean() > 0.5
    # dropping the last K block (with equal scales, so that no block dominates)
    one_a, one_b = np.full_like(asf, 127), np.full_like(bsf, 127)
    ref1 = mx.gemm(a, one_a, b, one_b)
    tol1 = mx.gemm_tolerance(a, one_a, b, one_b, np.float32(1), ref1)
    a2 = a.copy()
    a2[:, -16:] = 0
    bad = nv.bf16_to_f64(mx.gemm(a2, one_a, b, one_b))
    assert (np.abs(bad - nv.bf16_to_f64(ref1)) > tol1).mean() > 0.5
