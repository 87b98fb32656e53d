"""nvfp4_gemm_noalloc, the GEMM entry point that allocates nothing, against
nvfp4_gemm through the C ABI: the same bits on calls in a row (the second
smaller than the first, then the first again), each also within the oracle's
GEMM tolerance, and the host-side rejection of a plan whose scratch exceeds
the library's fixed array."""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_07_amd as nv
import synth
from tests.gpu_util import bits, check_gemm, dev, gpu_gemm, say, scalar

pytestmark = pytest.mark.gpu


def _operands(M, N, K, seed):
    a, b = synth.random_codes(seed, M, K), synth.random_codes(seed + 1, N, K)
    asf = synth.random_scale_bytes(seed + 2, M, K, lo=0x30, hi=0x40)
    bsf = synth.random_scale_bytes(seed + 3, N, K, lo=0x30, hi=0x40)
    return a, asf, b, bsf


def test_noalloc_matches_gemm_on_consecutive_calls():
    # split-K plans (their scratch is used): a K-group tile split five ways,
    # then a smaller register-tile call split two ways, then the first again
    # (the counters the earlier calls used must be back at zero); then a plan
    # with no split
    cases = [(1024, 256, 6144), (16, 768, 6144), (1024, 256, 6144), (64, 768, 1024)]
    for i, (M, N, K) in enumerate(cases):
        a, asf, b, bsf = _operands(M, N, K, 500 + 10 * i)
        at, asft, bt, bsft = dev(a), dev(asf), dev(b), dev(bsf)
        say("noalloc", i, M, N, K, nv.nvfp4_gemm_plan(M, N, K), nv.nvfp4_gemm_workspace_size(M, N, K))
        assert (nv.nvfp4_gemm_workspace_size(M, N, K) > 0) == (i < 3)
        want = bits(gpu_gemm(at, asft, bt, bsft, scalar(0.75), M, N, K))
        d = torch.full((M, N), 0x7FC1, dtype=torch.int16, device="cuda")
        nv.nvfp4_gemm_noalloc(at, asft, bt, bsft, scalar(0.75), d, M, N, K)
        got = bits(d)
        np.testing.assert_array_equal(got, want, err_msg=f"call {i}: {M}x{N}x{K}")
        check_gemm(got, a, asf, b, bsf, np.float32(0.75), f"noalloc {M}x{N}x{K}")


def test_noalloc_rejects_a_plan_beyond_its_scratch(force_plan):
    # 128x128 tiles forced to 16 splits at 1024 x 1024: 64 tiles x 16 x 64 KB
    # of partials, more than the 16 MiB array; rejected on the host
    M = N = 1024
    K = 6144
    force_plan(nv.FAMILY_GEMM, 1, 16)
    assert nv.nvfp4_gemm_workspace_size(M, N, K) > 16 << 20
    x = torch.zeros((M, K // 2), dtype=torch.uint8, device="cuda")
    s = torch.zeros((M, K // 16), dtype=torch.uint8, device="cuda")
    d = torch.zeros((M, N), dtype=torch.int16, device="cuda")
    with pytest.raises(nv.Nvfp4Error) as e:
        nv.nvfp4_gemm_noalloc(x, s, x, s, None, d, M, N, K)
    assert e.value.status == 5 and "scratch" in str(e.value)
    assert (bits(d) == 0).all()
