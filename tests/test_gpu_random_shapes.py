"""Seeded random shapes through the automatic plans, NVFP4 and MXFP4, every
output element compared with the oracle.  The shapes fall in four bands: decode
M (register tiles), mid M (split K-group LDS tiles, 128x128 tiles), large M x N
at small K (256x192 and 256x256 tiles, whole and partial rounds) and wide N at
small M, so the plan rules' boundaries and split counts are crossed at shapes
nobody chose by hand.  K is a multiple of 256 (the library's requirement); the
oracle's work is bounded by lowering K."""
import numpy as np
import pytest

import nvfp4_block_scaled_07_amd as nv
import synth
from tests.gpu_util import bits, check_gemm, dev, gpu_gemm, say, scalar
from tests.test_gpu_mx import _check as mx_check
from tests.test_gpu_mx import _mx_gemm
from tests.test_gpu_mx import _operands as mx_operands

MAX_FLOP = 4e10  # per shape, for the fp64 oracle


def random_shapes(seed, count):
    rng = np.random.default_rng(seed)
    shapes = []
    for i in range(count):
        band = i % 4
        if band == 0:
            M, N = int(rng.integers(1, 129)), int(rng.integers(1, 2561))
        elif band == 1:
            M, N = int(rng.integers(129, 1300)), int(rng.integers(64, 2561))
        elif band == 2:
            M, N = int(rng.integers(1800, 8400)), int(rng.integers(3000, 8400))
        else:
            M, N = int(rng.integers(1, 500)), int(rng.integers(2500, 12000))
        K = 256 * int(rng.integers(1, 25))
        while K > 256 and 2.0 * M * N * K > MAX_FLOP:
            K = max(256, (K // 2) // 256 * 256)
        shapes.append((M, N, K))
    return shapes


def test_the_bands_reach_every_automatic_plan_family():
    # host-side plan queries only
    plans = {nv.nvfp4_gemm_plan(*s) for s in random_shapes(2024, 32)}
    for family in ("kreg", "tile64x64k4", "tile256x192", "tile256x256"):
        assert any(p.startswith(family) for p in plans), (family, sorted(plans))


@pytest.mark.gpu
@pytest.mark.parametrize("M,N,K", random_shapes(2024, 32))
def test_nvfp4_random_shape(M, N, K):
    seed = 7 * M + 13 * N + K
    a, b = synth.random_codes(seed, M, K), synth.random_codes(seed + 1, N, K)
    asf = synth.random_scale_bytes(seed + 2, M, K, 0x28, 0x40)
    bsf = synth.random_scale_bytes(seed + 3, N, K, 0x28, 0x40)
    say("random nvfp4", M, N, K, nv.nvfp4_gemm_plan(M, N, K), nv.nvfp4_gemm_workspace_size(M, N, K))
    d = gpu_gemm(dev(a), dev(asf), dev(b), dev(bsf), scalar(0.5), M, N, K, d_fill=0x7FC1)
    check_gemm(bits(d), a, asf, b, bsf, np.float32(0.5), f"random {M}x{N}x{K}")


@pytest.mark.gpu
@pytest.mark.parametrize("M,N,K", random_shapes(2025, 16))
def test_mxfp4_random_shape(M, N, K):
    a, asf, b, bsf = mx_operands(3 * M + 5 * N + K, M, N, K)
    say("random mxfp4", M, N, K, nv.nvfp4_mx_gemm_plan(M, N, K), nv.nvfp4_mx_gemm_workspace_size(M, N, K))
    d = _mx_gemm(dev(a), dev(asf), dev(b), dev(bsf), scalar(0.5), M, N, K)
    mx_check(bits(d), a, asf, b, bsf, np.float32(0.5), f"random mx {M}x{N}x{K}")
