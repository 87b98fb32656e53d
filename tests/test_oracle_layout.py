"""Pins of the oracle's 128 x 4 tiled scale layout (CPU): a hand-placed tile,
the same layout written as a reshape and axis permutation of the padded
matrix, and the round trip on ragged shapes."""
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
