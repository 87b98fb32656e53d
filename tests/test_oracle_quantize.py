"""Pins for the oracle's quantiser (CPU only): closed forms, round trips and
invariants that the block-scaling rule fixes."""
import numpy as np
import pytest

from oracle import nvfp4_ref as o


def _codes(q):
    return o.unpack_codes(q)


def test_on_grid_block_with_amax_six_is_exact():
    # amax = 6 and gs = 1 give t = 1 -> scale 0x38, r = 1, so every code is exact
    x = np.zeros((1, 16), np.float32)
    x[0, :8] = [6, -4, 3, 0.5, 0, -1.5, 2, -6]
    q, sf = o.quantize(x, np.float32(1))
    assert sf.tolist() == [[0x38]]
    assert _codes(q)[0, :8].tolist() == [0x7, 0xE, 0x5, 0x1, 0x0, 0xB, 0x4, 0xF]
    # packing: element 0 in the low nibble of byte 0
    assert int(q[0, 0]) == (0x7 | (0xE << 4))


def test_zero_block_gives_zero_scale_and_zero_codes():
    x = np.zeros((2, 32), np.float32)
    x[1, 16:] = 1.0
    q, sf = o.quantize(x, np.float32(1))
    assert sf[0].tolist() == [0, 0] and sf[1, 0] == 0
    assert (_codes(q)[0] == 0).all()


def test_scale_is_amax_over_six_times_gs():
    # amax 3 -> t = 0.5 -> 0x30 ; gs = 4 -> t = 2 -> 0x40 ; values then land on the grid
    x = np.zeros((1, 16), np.float32)
    x[0, 0] = 3.0
    x[0, 1] = -1.5
    q, sf = o.quantize(x, np.float32(1))
    assert sf[0, 0] == 0x30 and _codes(q)[0, :2].tolist() == [0x7, 0xD]
    q, sf = o.quantize(x, np.float32(4))
    assert sf[0, 0] == 0x40 and _codes(q)[0, :2].tolist() == [0x7, 0xD]


def test_scale_saturates_at_448():
    x = np.full((1, 16), 1e6, np.float32)
    q, sf = o.quantize(x, np.float32(1))
    assert sf[0, 0] == 0x7E and (_codes(q) == 0x7).all()


def test_negative_zero_and_negative_underflow_keep_sign():
    x = np.zeros((1, 16), np.float32)
    x[0, 0] = 6.0
    x[0, 1] = -0.1     # rounds to zero magnitude with sign kept
    x[0, 2] = -0.0
    q, sf = o.quantize(x, np.float32(1))
    assert _codes(q)[0, :3].tolist() == [0x7, 0x8, 0x8]


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_round_trip_of_representable_blocks(seed):
    # blocks whose dequantised values contain +-6 * s quantise back to (q, s)
    rng = np.random.default_rng(seed)
    R, K = 64, 256
    codes = rng.integers(0, 16, size=(R, K)).astype(np.uint8)
    codes[:, ::16] = rng.choice([0x7, 0xF], size=(R, K // 16))   # one +-6 per block
    q = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    sf = rng.integers(1, 0x7F, size=(R, K // 16)).astype(np.uint8)
    x = o.dequant(q, sf).astype(np.float32)
    q2, sf2 = o.quantize(x, np.float32(1))
    np.testing.assert_array_equal(sf2, sf)
    np.testing.assert_array_equal(q2, q)


def test_power_of_two_input_scaling_shifts_only_the_scales():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((32, 128)).astype(np.float32)
    q1, s1 = o.quantize(x, np.float32(1))
    q2, s2 = o.quantize(x * np.float32(4), np.float32(1))
    q3, s3 = o.quantize(x, np.float32(4))
    np.testing.assert_array_equal(q1, q2)
    np.testing.assert_array_equal(q1, q3)
    np.testing.assert_array_equal(s3, s2)
    # normal-range scales move up by exactly 2 exponent steps (+16 in the byte)
    normal = (s1 >= 0x08) & (s1 <= 0x6E)
    np.testing.assert_array_equal(s2[normal].astype(int), s1[normal].astype(int) + 16)


def test_dequantisation_error_is_within_half_a_grid_step():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((64, 512)).astype(np.float32)
    gs = o.global_encode_scale(x)
    q, sf = o.quantize(x, gs)
    xh = o.dequant(q, sf) / np.float64(gs)
    sv = np.repeat(o.E4M3_LUT[sf], 16, axis=1) / np.float64(gs)
    # grid step around |y| (y = x / sv) is 0.5 below 2, 1 below 4, 2 above
    y = np.abs(x.astype(np.float64)) / sv
    half = np.where(y < 2, 0.25, np.where(y < 4, 0.5, 1.0))
    err = np.abs(xh - x)
    assert (err <= half * sv * (1 + 1e-6) + 1e-30).all()


def test_global_scale_and_alpha():
    x = np.array([[0.5, -3.0, 2.0]], np.float32)
    assert o.global_encode_scale(x) == np.float32(2688.0 / 3.0)
    assert o.global_encode_scale(np.zeros((2, 2), np.float32)) == np.float32(1)
    gs_a, gs_b = np.float32(896.0), np.float32(0.5)
    assert o.alpha_from_scales(gs_a, gs_b) == np.float32(1.0 / 448.0)


def test_quantize_rejects_bad_shapes():
    with pytest.raises(ValueError):
        o.quantize(np.zeros((2, 20), np.float32))
