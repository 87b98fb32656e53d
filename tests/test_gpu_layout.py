"""GPU parity of the scale-layout interop calls (128 x 4 tiles), through the
C ABI: bytes equal to the oracle's on ragged shapes, the round trip, and a
GEMM on scales imported from the tiled layout."""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_07_amd as nv
import synth
from oracle import nvfp4_ref as o
from tests.gpu_util import bits, check_gemm, dev, gpu_gemm, host, say, scalar

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("rows,K", [(1, 16), (130, 80), (300, 6144), (257, 1040)])
def test_tiled_layout_bytes_and_round_trip(rows, K):
    sf = np.random.default_rng(rows + K).integers(0, 256, (rows, K // 16), dtype=np.uint8)
    n = nv.nvfp4_scales_128x4_size(rows, K)
    assert n == o.tiled128x4_size(rows, K)
    say("tiled layout", rows, K)
    tiled = torch.full((n,), 0xAB, dtype=torch.uint8, device="cuda")
    nv.nvfp4_scales_to_128x4(dev(sf), tiled, rows, K)
    np.testing.assert_array_equal(host(tiled), o.scales_to_128x4(sf))
    back = torch.empty((rows, K // 16), dtype=torch.uint8, device="cuda")
    nv.nvfp4_scales_from_128x4(dev(o.scales_to_128x4(sf)), back, rows, K)
    np.testing.assert_array_equal(host(back), sf)


def test_gemm_on_imported_scales():
    M, N, K = 200, 330, 1536
    a, b = synth.random_codes(151, M, K), synth.random_codes(152, N, K)
    asf = synth.random_scale_bytes(153, M, K, lo=0x28, hi=0x48)
    bsf = synth.random_scale_bytes(154, N, K, lo=0x28, hi=0x48)
    say("gemm on imported scales")
    asf_t = torch.empty((M, K // 16), dtype=torch.uint8, device="cuda")
    bsf_t = torch.empty((N, K // 16), dtype=torch.uint8, device="cuda")
    nv.nvfp4_scales_from_128x4(dev(o.scales_to_128x4(asf)), asf_t, M, K)
    nv.nvfp4_scales_from_128x4(dev(o.scales_to_128x4(bsf)), bsf_t, N, K)
    d = gpu_gemm(dev(a), asf_t, dev(b), bsf_t, scalar(0.5), M, N, K)
    check_gemm(bits(d), a, asf, b, bsf, np.float32(0.5), "imported scales")
