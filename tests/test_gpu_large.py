"""Full-output GPU parity of the large compute-bound GEMMs (M = 2048, 4096,
8192, 16384 x N = 6144 x K = 6144), NVFP4 and MXFP4, through the C ABI.  The
four M values take four different automatic plans on each path (NVFP4: one
round of 256x192 tiles, two rounds of them, 256x256 tiles; MXFP4: 256x256 tiles
at three quarters of a round, 256x192, 256x256).

Every element of every output is compared with the oracle: the oracle runs
on row blocks in a pool of CPU processes (rows of a GEMM are independent), and
the M values share one oracle evaluation because the workload's sweep is
nested (A is drawn at M = 16384 and the smaller M take its first rows)."""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_07_amd as nv
import synth
from oracle import nvfp4_ref as o
from tests import oracle_pool as op
from tests.gpu_util import bits, dev, gpu_global_scale, gpu_quantize, host, say

pytestmark = pytest.mark.gpu

MS = (2048, 4096, 8192, 16384)
N = K = 6144
BLOCK = 1024


def _compare_blocks(pool, fmt, qa, sfa, qb, sfb, alpha, outs):
    """Stats per output (outs: M -> bf16 bits [M][N]) over 1024-row blocks;
    each block's oracle is evaluated once for every output that covers it."""
    jobs, cover = [], []
    for r0 in range(0, max(outs), BLOCK):
        r1 = r0 + BLOCK
        ms = [m for m in sorted(outs) if m >= r1]
        cover.append(ms)
        jobs.append((fmt, qa[r0:r1], sfa[r0:r1], qb, sfb, alpha, [outs[m][r0:r1] for m in ms]))
    stats = {m: op.Stats() for m in outs}
    for ms, res in zip(cover, pool.imap(op.gemm_rows_compare, jobs)):
        for m, st in zip(ms, res):
            stats[m].add(st)
    return stats


@pytest.mark.timeout(900)
def test_large_nvfp4_full_output_every_m():
    name = "large_n6144_k6144"
    say("large: inputs")
    a, b = synth.single_operands(name, max(MS))
    gsa, gsb = o.global_encode_scale(a), o.global_encode_scale(b)
    alpha = o.alpha_from_scales(gsa, gsb)
    with op.make_pool() as pool:
        # the oracle's bytes (row blocks in the pool) while the GPU quantises
        qa_jobs = pool.map_async(op.quantize_block, [(a[r:r + BLOCK], gsa) for r in range(0, a.shape[0], BLOCK)])
        qb_jobs = pool.map_async(op.quantize_block, [(b[r:r + BLOCK], gsb) for r in range(0, b.shape[0], BLOCK)])
        at, bt = dev(a), dev(b)
        gsa_t, gsb_t = gpu_global_scale(at), gpu_global_scale(bt)
        assert host(gsa_t)[0] == gsa and host(gsb_t)[0] == gsb
        alpha_t = torch.empty(1, dtype=torch.float32, device="cuda")
        nv.nvfp4_alpha_from_scales(gsa_t, gsb_t, alpha_t, 1)
        assert host(alpha_t)[0] == alpha
        qa_t, sfa_t = gpu_quantize(at, gsa_t)
        qb_t, sfb_t = gpu_quantize(bt, gsb_t)
        del at, bt
        outs = {}
        for m in MS:
            say("large nvfp4 M =", m, "plan", nv.nvfp4_gemm_plan(m, N, K))
            d = torch.empty((m, N), dtype=torch.int16, device="cuda")
            nv.nvfp4_gemm(qa_t[:m], sfa_t[:m], qb_t, sfb_t, alpha_t, d, m, N, K, nv.gemm_workspace(m, N, K))
            outs[m] = bits(d)
            del d
        say("large: oracle quantisation")
        qa = np.concatenate([q for q, _ in qa_jobs.get()])
        sfa = np.concatenate([s for _, s in qa_jobs.get()])
        qb = np.concatenate([q for q, _ in qb_jobs.get()])
        sfb = np.concatenate([s for _, s in qb_jobs.get()])
        np.testing.assert_array_equal(host(qa_t), qa)
        np.testing.assert_array_equal(host(sfa_t), sfa)
        np.testing.assert_array_equal(host(qb_t), qb)
        np.testing.assert_array_equal(host(sfb_t), sfb)
        del qa_t, sfa_t, qb_t, sfb_t
        say("large: oracle GEMM, every element")
        stats = _compare_blocks(pool, "nv", qa, sfa, qb, sfb, alpha, outs)
    for m in MS:
        st = stats[m].check(f"nvfp4 {m}x{N}x{K}")
        assert st.n == m * N
        say(f"M={m}: {st.n} elements, frob {st.frob:.3g}, strict 2-ulp {st.strict / st.n:.6f}")


SCALE_LO, SCALE_HI = 120, 134   # E8M0 bytes: 2**-7 .. 2**7


@pytest.mark.timeout(900)
def test_large_mxfp4_full_output_every_m():
    mmax = max(MS)
    a, b = synth.random_codes(7300, mmax, K), synth.random_codes(7301, N, K)
    asf = synth.random_scale_bytes(7302, mmax, 2 * K, SCALE_LO, SCALE_HI)[:, : K // 32].copy()
    bsf = synth.random_scale_bytes(7303, N, 2 * K, SCALE_LO, SCALE_HI)[:, : K // 32].copy()
    alpha = np.float32(0.5)
    at, asft, bt, bsft = dev(a), dev(asf), dev(b), dev(bsf)
    alpha_t = torch.tensor([alpha], dtype=torch.float32, device="cuda")
    outs = {}
    for m in MS:
        say("large mxfp4 M =", m, "plan", nv.nvfp4_mx_gemm_plan(m, N, K))
        d = torch.empty((m, N), dtype=torch.int16, device="cuda")
        nv.nvfp4_mx_gemm(at[:m], asft[:m], bt, bsft, alpha_t, d, m, N, K, nv.mx_gemm_workspace(m, N, K))
        outs[m] = bits(d)
        del d
    with op.make_pool() as pool:
        say("large mxfp4: oracle GEMM, every element")
        stats = _compare_blocks(pool, "mx", a, asf, b, bsf, alpha, outs)
    for m in MS:
        st = stats[m].check(f"mxfp4 {m}x{N}x{K}")
        assert st.n == m * N
        say(f"MX M={m}: {st.n} elements, frob {st.frob:.3g}, strict 2-ulp {st.strict / st.n:.6f}")
