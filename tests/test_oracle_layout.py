"""Pins of the oracle's tiled scale layouts, 128 x 4 and 8 x 4 (CPU): a
hand-placed tile, the same layout written as a reshape and axis permutation
of the padded matrix, and the round trip on ragged shapes.  Both layouts are
readings (the pages only name the switch between layouts), so these pins
catch index slips, not a wrong reading: parity unpinned."""
import numpy as np

from oracle import nvfp4_ref as o


def test_hand_placed_entries_of_one_tile():
    sf = np.zeros((128, 4), np.uint8)
    sf[0, 0], sf[1, 0], sf[0, 1], sf[32, 0], sf[127, 3] = 1, 2, 3, 4, 5
    t = o.scales_to_128x4(sf)
    assert t.size == 512
    assert t[0] == 1 and t[16] == 2 and t[1] == 3 and t[4] == 4
    assert t[31 * 16 + 3 * 4 + 3] == 5


def test_reshape_form_and_round_trip():
    rng = np.random.default_rng(5)
    for rows, K in [(1, 16), (128, 64), (130, 80), (300, 6144), (257, 1040)]:
        cols = K // 16
        sf = rng.integers(0, 256, (rows, cols), dtype=np.uint8)
        t = o.scales_to_128x4(sf)
        assert t.size == o.tiled128x4_size(rows, K)
        # the same layout as a reshape of the zero-padded matrix:
        # [tiles_r][4][32][tiles_c][4] -> [tiles_r][tiles_c][32][4][4]
        R, C = -(-rows // 128) * 128, -(-cols // 4) * 4
        pad = np.zeros((R, C), np.uint8)
        pad[:rows, :cols] = sf
        ref = pad.reshape(R // 128, 4, 32, C // 4, 4).transpose(0, 3, 2, 1, 4).reshape(-1)
        np.testing.assert_array_equal(t, ref)
        np.testing.assert_array_equal(o.scales_from_128x4(t, rows, K), sf)


def test_8x4_hand_placed_entries():
    sf = np.zeros((9, 6), np.uint8)
    sf[0, 0], sf[0, 1], sf[1, 0], sf[7, 3], sf[0, 4], sf[8, 0], sf[8, 5] = 1, 2, 3, 4, 5, 6, 7
    t = o.scales_to_8x4(sf)
    assert t.size == 16 * 8 == o.tiled8x4_size(9, 96)     # 2 x 2 tiles of 32 bytes
    assert t[0] == 1 and t[1] == 2 and t[4] == 3 and t[7 * 4 + 3] == 4
    assert t[32] == 5                                      # tile (0, 1), row 0, column 0
    assert t[64] == 6 and t[96 + 1] == 7                   # tiles (1, 0) and (1, 1)
    assert t[32 + 2] == 0 and t[96 + 2] == 0               # padding columns 6, 7


def test_8x4_reshape_form_and_round_trip():
    rng = np.random.default_rng(6)
    for rows, K in [(1, 16), (8, 64), (9, 80), (300, 6144), (257, 1040)]:
        cols = K // 16
        sf = rng.integers(0, 256, (rows, cols), dtype=np.uint8)
        t = o.scales_to_8x4(sf)
        assert t.size == o.tiled8x4_size(rows, K)
        R, C = -(-rows // 8) * 8, -(-cols // 4) * 4
        pad = np.zeros((R, C), np.uint8)
        pad[:rows, :cols] = sf
        # [tiles_r][8][tiles_c][4] -> [tiles_r][tiles_c][8][4]
        ref = pad.reshape(R // 8, 8, C // 4, 4).transpose(0, 2, 1, 3).reshape(-1)
        np.testing.assert_array_equal(t, ref)
        np.testing.assert_array_equal(o.scales_from_8x4(t, rows, K), sf)
