"""Seeded random grouped GEMMs through the automatic grouped plans, on plain
[E][N][K/2] weights and on packed weights: random expert counts, random row
distributions (empty experts, experts past 64 rows, rows past offsets[E] that
must stay untouched), ragged N and K any multiple of 256 (the plain kernel's
fallback takes odd multiples).  Every expert's rows are compared with the
oracle, and, where K allows packing (a multiple of 512), the packed call bit
for bit with the plain one."""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_07_amd as nv
import synth
from tests.gpu_util import bits, check_gemm, dev, host, say

SENTINEL = 0x7FC1


def random_grouped_cases(seed, count):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(count):
        E = int(rng.integers(1, 41))
        routed = int(rng.integers(1, 64 * E + 2))
        routed = min(routed, 1500)
        cuts = np.sort(rng.integers(0, routed + 1, size=E - 1))
        off = np.concatenate([[0], cuts, [routed]]).astype(np.int32)
        tail = int(rng.integers(0, 3)) * int(rng.integers(1, 40))  # rows past offsets[E]
        N = int(rng.integers(1, 1201))
        K = 256 * int(rng.integers(1, 13))
        cases.append((seed * 100 + i, E, off, routed + tail, N, K))
    return cases


CASES = random_grouped_cases(31, 12)


def test_random_cases_cover_empty_and_tall_experts():
    # host-side only: the sweep has empty experts and experts past 64 rows,
    # and both the 32-row and the 64-row pass plans
    sizes = np.concatenate([np.diff(c[2]) for c in CASES])
    assert (sizes == 0).any() and (sizes > 64).any()
    tall = [c[2][-1] > 40 * c[1] for c in CASES]
    assert any(tall) and not all(tall)
    assert any(c[5] % 512 for c in CASES) and any(c[5] % 512 == 0 for c in CASES)


@pytest.mark.gpu
@pytest.mark.parametrize("case", range(len(CASES)))
def test_random_grouped_plain_and_packed(case):
    seed, E, off, rows, N, K = CASES[case]
    a = synth.random_codes(seed + 1, rows, K)
    asf = synth.random_scale_bytes(seed + 2, rows, K, lo=0x30, hi=0x40)
    b = synth.random_codes(seed + 3, E * N, K).reshape(E, N, K // 2)
    bsf = synth.random_scale_bytes(seed + 4, E * N, K, lo=0x30, hi=0x40).reshape(E, N, K // 16)
    alpha = np.random.default_rng(seed + 5).uniform(0.25, 2.0, E).astype(np.float32)
    say("grouped random", case, "E", E, "rows", rows, "routed", int(off[-1]), "N", N, "K", K,
        "max rows/expert", int(np.diff(off).max()))
    a_t, asf_t, b_t, bsf_t, off_t, al_t = dev(a), dev(asf), dev(b), dev(bsf), dev(off), dev(alpha)
    d = torch.full((rows, N), SENTINEL, dtype=torch.int16, device="cuda")
    st = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    need = nv.nvfp4_grouped_workspace_size(rows, N, K, E)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda") if need else None
    nv.nvfp4_grouped_gemm(a_t, asf_t, b_t, bsf_t, off_t, al_t, d, rows, N, K, E, ws, st)
    assert int(host(st)[0]) == 0
    db = bits(d)
    for e in range(E):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi > lo:
            check_gemm(db[lo:hi], a[lo:hi], asf[lo:hi], b[e], bsf[e], alpha[e], f"case {case} expert {e}")
    assert (db[int(off[-1]):] == SENTINEL).all()
    if K % 512:
        return  # packed weights need whole 512-element stage pairs
    pb, psf = nv.grouped_pack(b_t, bsf_t, N, K, E)
    d2 = torch.full((rows, N), SENTINEL, dtype=torch.int16, device="cuda")
    nv.nvfp4_grouped_gemm_packed(a_t, asf_t, pb, psf, off_t, al_t, d2, rows, N, K, E, st)
    assert int(host(st)[0]) == 0
    np.testing.assert_array_equal(bits(d2), db)
