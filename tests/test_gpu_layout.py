"""GPU parity of the scale-layout interop calls (128 x 4 and 8 x 4 tiles),
through the C ABI: bytes equal to the oracle's on ragged shapes, the round
trip, and a GEMM on scales imported from each tiled layout."""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_07_amd as nv
import synth
from oracle import nvfp4_ref as o
from tests.gpu_util import bits, check_gemm, dev, gpu_gemm, host, say, scalar

pytestmark = pytest.mark.gpu


LAYOUTS = {
    "128x4": (nv.nvfp4_scales_128x4_size, nv.nvfp4_scales_to_128x4, nv.nvfp4_scales_from_128x4,
              o.tiled128x4_size, o.scales_to_128x4, o.scales_from_128x4),
    "8x4": (nv.nvfp4_scales_8x4_size, nv.nvfp4_scales_to_8x4, nv.nvfp4_scales_from_8x4,
            o.tiled8x4_size, o.scales_to_8x4, o.scales_from_8x4),
}


@pytest.mark.parametrize("layout", ["128x4", "8x4"])
@pytest.mark.parametrize("rows,K", [(1, 16), (9, 80), (130, 80), (300, 6144), (257, 1040), (4096, 6144)])
def test_tiled_layout_bytes_and_round_trip(layout, rows, K):
    size, to_t, from_t, o_size, o_to, _ = LAYOUTS[layout]
    sf = np.random.default_rng(rows + K).integers(0, 256, (rows, K // 16), dtype=np.uint8)
    n = size(rows, K)
    assert n == o_size(rows, K)
    say("tiled layout", layout, rows, K)
    tiled = torch.full((n,), 0xAB, dtype=torch.uint8, device="cuda")
    to_t(dev(sf), tiled, rows, K)
    np.testing.assert_array_equal(host(tiled), o_to(sf))
    back = torch.empty((rows, K // 16), dtype=torch.uint8, device="cuda")
    from_t(dev(o_to(sf)), back, rows, K)
    np.testing.assert_array_equal(host(back), sf)


@pytest.mark.parametrize("layout", ["128x4", "8x4"])
def test_gemm_on_imported_scales(layout):
    _, _, from_t, _, o_to, _ = LAYOUTS[layout]
    M, N, K = 200, 330, 1536
    a, b = synth.random_codes(151, M, K), synth.random_codes(152, N, K)
    asf = synth.random_scale_bytes(153, M, K, lo=0x28, hi=0x48)
    bsf = synth.random_scale_bytes(154, N, K, lo=0x28, hi=0x48)
    say("gemm on imported scales", layout)
    asf_t = torch.empty((M, K // 16), dtype=torch.uint8, device="cuda")
    bsf_t = torch.empty((N, K // 16), dtype=torch.uint8, device="cuda")
    from_t(dev(o_to(asf)), asf_t, M, K)
    from_t(dev(o_to(bsf)), bsf_t, N, K)
    d = gpu_gemm(dev(a), asf_t, dev(b), bsf_t, scalar(0.5), M, N, K)
    check_gemm(bits(d), a, asf, b, bsf, np.float32(0.5), "imported scales")


# nvfp4_gemm_sf: register-tile plans read the tiled scales in place (M <= 128
# here), every other plan converts them into the workspace first.
SF_CASES = [(1, 200, 512), (16, 768, 6144), (33, 130, 1024), (64, 2048, 2304), (128, 320, 768),
            (16, 16384, 1024), (130, 300, 1280), (1000, 768, 2048), (2048, 6144, 512)]


@pytest.mark.parametrize("layout", ["128x4", "8x4"])
@pytest.mark.parametrize("M,N,K", SF_CASES)
def test_gemm_on_tiled_scales(layout, M, N, K):
    _, _, _, _, o_to, _ = LAYOUTS[layout]
    sfl = nv.SF_128x4 if layout == "128x4" else nv.SF_8x4
    seed = 17 * M + N + K
    a, b = synth.random_codes(seed, M, K), synth.random_codes(seed + 1, N, K)
    asf = synth.random_scale_bytes(seed + 2, M, K, lo=0x28, hi=0x48)
    bsf = synth.random_scale_bytes(seed + 3, N, K, lo=0x28, hi=0x48)
    plan = nv.nvfp4_gemm_plan(M, N, K)
    need = nv.nvfp4_gemm_sf_workspace_size(M, N, K, sfl)
    say("gemm on tiled scales", layout, M, N, K, plan, need)
    ws = nv.nvfp4_workspace_init(torch.empty(need, dtype=torch.uint8, device="cuda")) if need else None
    a_t, b_t = dev(a), dev(b)
    alpha = scalar(0.75)
    d = torch.full((M, N), 0x7FC1, dtype=torch.int16, device="cuda")
    nv.nvfp4_gemm_sf(a_t, dev(o_to(asf)), b_t, dev(o_to(bsf)), alpha, d, M, N, K, sfl, ws)
    # bit for bit the call on linear scales, and within tolerance of the oracle
    ref = gpu_gemm(a_t, dev(asf), b_t, dev(bsf), alpha, M, N, K)
    np.testing.assert_array_equal(bits(d), bits(ref), err_msg=f"{layout} {M}x{N}x{K} ({plan})")
    check_gemm(bits(d), a, asf, b, bsf, np.float32(0.75), f"tiled scales {layout} {M}x{N}x{K}")
    if ws is not None:   # the workspace serves a second call (counters left at zero)
        d2 = torch.zeros_like(d)
        nv.nvfp4_gemm_sf(a_t, dev(o_to(asf)), b_t, dev(o_to(bsf)), alpha, d2, M, N, K, sfl, ws)
        np.testing.assert_array_equal(bits(d2), bits(d))


def test_tiled_scale_cases_reach_both_paths():
    # host-side: the cases cover plans that read in place and plans that convert
    plans = [nv.nvfp4_gemm_plan(M, N, K) for M, N, K in SF_CASES]
    assert any(p.startswith("kreg") for p in plans) and any(not p.startswith("kreg") for p in plans)
