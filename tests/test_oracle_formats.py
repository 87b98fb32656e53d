"""Pins for the oracle's code tables and rounding (CPU only).

Each check compares the oracle with something other than itself: the golden
tables under tests/golden (values fixed by the format definitions), torch's
CPU float8_e4m3fn decode and cast (a library routine), and torch's fp32->bf16
cast.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import nvfp4_ref as o

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def test_e2m1_table_matches_golden():
    g = _load("e2m1_codes.json")["values"]
    for code in range(16):
        want = g[str(code)]
        got = o.E2M1_LUT[code]
        assert got == want and math.copysign(1, got) == math.copysign(1, want), code


def test_e4m3_decode_matches_torch_all_codes():
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = o.E4M3_LUT
    nan_t, nan_o = np.isnan(t), np.isnan(ours)
    assert (nan_t == nan_o).all()
    assert nan_o.sum() == 2 and nan_o[0x7F] and nan_o[0xFF]
    np.testing.assert_array_equal(ours[~nan_o], t[~nan_t])
    assert (np.signbit(ours[~nan_o]) == np.signbit(t[~nan_t])).all()


def test_e4m3_anchors():
    g = _load("e4m3_anchors.json")["anchors"]
    for k, v in g.items():
        got = o.E4M3_LUT[int(k, 16)]
        if v == "nan":
            assert math.isnan(got)
        else:
            assert got == v and math.copysign(1, got) == math.copysign(1, v), k


def _torch_e4m3(t):
    """torch CPU cast (round to nearest even, no saturation) on inputs clamped to 448."""
    tt = torch.from_numpy(np.minimum(np.abs(t), 448.0).astype(np.float32) * np.where(np.signbit(t), -1, 1).astype(np.float32))
    return tt.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_encode_matches_torch_on_values_midpoints_and_random():
    pos = o.E4M3_LUT[:0x7F]
    mids = (pos[:-1] + pos[1:]) / 2            # exact ties (exact in fp32)
    rng = np.random.default_rng(7)
    rnd = np.concatenate([rng.uniform(0, 500, 20000), np.exp(rng.uniform(-16, 7, 20000))])
    for arr in (pos, mids, rnd, -mids):
        t = np.asarray(arr, dtype=np.float32)
        np.testing.assert_array_equal(o.e4m3_encode(t), _torch_e4m3(t))


def test_e4m3_encode_hand_ties_and_saturation():
    cases = {464.0: 0x7E, 480.0: 0x7E, 1e9: 0x7E, 2.0 ** -10: 0x00, 3 * 2.0 ** -11: 0x01,
             1.0625: 0x38, 1.0625 + 2 ** -20: 0x39, 0.0: 0x00}
    for t, want in cases.items():
        assert int(o.e4m3_encode(np.float32(t))) == want, t


def test_e2m1_rounding_golden():
    g = _load("e2m1_rounding.json")["cases"]
    for y, want in g:
        assert int(o.e2m1_encode(np.float32(y))) == want, y


def test_e2m1_encode_round_trip_and_monotone():
    # every code maps back to itself, and encoding is monotone in |y|
    for c in range(16):
        v = np.float32(o.E2M1_LUT[c])
        if c == 8:
            v = np.float32(-0.0)
        assert int(o.e2m1_encode(v)) == c
    ys = np.sort(np.abs(np.random.default_rng(3).uniform(0, 8, 50000))).astype(np.float32)
    codes = o.e2m1_encode(ys)
    assert (np.diff(codes.astype(int)) >= 0).all()


def test_bf16_rne_matches_torch_on_fp32_inputs():
    rng = np.random.default_rng(11)
    x = np.concatenate([rng.standard_normal(100000) * 10.0 ** rng.uniform(-30, 30, 100000),
                        [0.0, -0.0, 1.0, 3.0e38, -3.0e38]]).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = o.bf16_rne(x.astype(np.float64))
    np.testing.assert_array_equal(got, want)


def test_bf16_rne_hand_cases_single_rounding():
    # 1 + 2^-8 is a tie -> 1.0 ; 1 + 3*2^-8 is a tie -> 1 + 2^-6 (even);
    # 1 + 2^-8 + 2^-40 is above the tie: direct rounding gives 1 + 2^-7
    # (rounding through fp32 first would give 1.0).
    cases = [(1 + 2 ** -8, 1.0), (1 + 3 * 2 ** -8, 1 + 2 ** -6), (1 + 2 ** -8 + 2 ** -40, 1 + 2 ** -7),
             (-(1 + 2 ** -8 + 2 ** -40), -(1 + 2 ** -7)), (8064.21875, 8064.0)]
    for x, want in cases:
        got = o.bf16_to_f64(o.bf16_rne(np.array([x])))[0]
        assert got == want, (x, got, want)


# The only output figures the pages print (P1 "The Results: A Correction":
# abs_max 18743296 and abs_mean 626688 for M = 128, N = 256, K = 256 with
# random scale bytes).  Their inputs are not printed, so they pin nothing of
# the oracle; they are exact bf16 numbers, as a bf16 output implies.
PAGE_SMOKE_MAGNITUDES = (18743296.0, 626688.0)


def test_page_printed_outputs_are_bf16_values():
    for v in PAGE_SMOKE_MAGNITUDES:
        assert o.bf16_to_f64(o.bf16_rne(np.array([v])))[0] == v
