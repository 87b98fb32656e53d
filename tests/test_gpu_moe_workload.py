"""The grouped MoE workload as stated, every expert, through the C ABI.

512 tokens of N(0, 1) activations routed top-8 over 256 experts by a seeded
softmax over N(0, 1) logits (4096 rows, rows ordered by expert then token);
each expert's [2048][6144] weights drawn N(0, 0.02) and quantised on their own,
with the expert's encode scale gs_e and alpha[e] = 1 / (gs_a * gs_e) (pages
"When a Benchmark Crashes: The Elusive FP4 GEMM Comparison on Blackwell
SM120", section "Why This Message Was Written": 256 experts, 8 active, hidden
size 6144, expert intermediate size 2048).

Checked, on the GPU against the oracle:
* the quantisation of every expert's weights (bytes), its encode scale and
  alpha (bits), and of the activations;
* every row of every expert of nvfp4_grouped_gemm ([E][N][K/2] weights),
  nvfp4_grouped_gemm_packed (the same weights packed) and
  nvfp4_grouped_gemm_packed_fused (bf16 token activations gathered and
  quantised inside the GEMM), element by element at the GEMM tolerance.
The oracle runs one expert per task in a pool of CPU processes."""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import nvfp4_block_scaled_07_amd as nv
import synth
from oracle import nvfp4_ref as o
from tests import oracle_pool as op
from tests.gpu_util import bits, dev, gpu_global_scale, gpu_quantize, host, say

pytestmark = pytest.mark.gpu
SENTINEL = 0x7FC1


def _bf16_bits(x32: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of fp32 values, round to nearest even (torch's CPU cast)."""
    return torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.timeout(1200)
def test_grouped_moe_workload_as_stated_every_expert():
    g = synth.GROUPED
    T, E, N, K, k = g["tokens"], g["experts"], g["n"], g["k"], g["top_k"]
    tok, off = synth.routing(g["seed_router"], T, E, k)
    rows = int(off[-1])
    assert rows == T * k
    say("moe workload: activations")
    x = synth.token_activations(T, K)
    gsa = o.global_encode_scale(x)
    qa_tok, sfa_tok = o.quantize(x, gsa)
    xt = dev(x)
    gsa_t = gpu_global_scale(xt)
    assert host(gsa_t)[0] == gsa
    qa_t_tok, sfa_t_tok = gpu_quantize(xt, gsa_t)
    np.testing.assert_array_equal(host(qa_t_tok), qa_tok)
    np.testing.assert_array_equal(host(sfa_t_tok), sfa_tok)
    # the fused path reads the same tokens as bf16 and quantises them with
    # the same (static) activation scale
    xb = _bf16_bits(x)
    qf_tok, sff_tok = o.quantize(o.bf16_bits_to_f32(xb), gsa)
    tok_t = torch.from_numpy(tok).cuda()
    qa_t, sfa_t = qa_t_tok[tok_t].contiguous(), sfa_t_tok[tok_t].contiguous()

    b_t = torch.empty((E, N, K // 2), dtype=torch.uint8, device="cuda")
    bsf_t = torch.empty((E, N, K // 16), dtype=torch.uint8, device="cuda")
    gs_e = np.zeros(E, np.float32)
    alpha = np.zeros(E, np.float32)
    oracle_rows = {}
    jobs = []
    for e in range(E):
        rt = tok[off[e]:off[e + 1]]
        jobs.append((e, gsa, [(qa_tok[rt], sfa_tok[rt]), (qf_tok[rt], sff_tok[rt])], N, K))
    say("moe workload: 256 experts' weights, oracle and GPU quantisation")
    q_t = torch.empty((N, K // 2), dtype=torch.uint8, device="cuda")
    sf_t = torch.empty((N, K // 16), dtype=torch.uint8, device="cuda")
    ahead = 16                         # fp32 weights generated ahead of their turn
    with op.make_pool() as pool, ThreadPoolExecutor(4) as threads:
        weights = {e: threads.submit(synth.expert_weights, e, N, K) for e in range(min(ahead, E))}
        for e, qb, sfb, gs, al, res in pool.imap(op.expert_oracle, jobs):
            wt = dev(weights.pop(e).result())
            if e + ahead < E:
                weights[e + ahead] = threads.submit(synth.expert_weights, e + ahead, N, K)
            gs_t = gpu_global_scale(wt)
            assert host(gs_t)[0] == gs, f"expert {e}: encode scale"
            nv.nvfp4_quantize(wt, N, K, gs_t, q_t, sf_t)
            np.testing.assert_array_equal(host(q_t), qb, err_msg=f"expert {e}: codes")
            np.testing.assert_array_equal(host(sf_t), sfb, err_msg=f"expert {e}: scales")
            b_t[e].copy_(torch.from_numpy(qb))
            bsf_t[e].copy_(torch.from_numpy(sfb))
            gs_e[e], alpha[e] = gs, al
            oracle_rows[e] = res
            if e % 32 == 0:
                say("expert", e, "rows", int(off[e + 1] - off[e]))
    alpha_t = torch.empty(E, dtype=torch.float32, device="cuda")
    nv.nvfp4_alpha_from_scales(gsa_t, dev(gs_e), alpha_t, E)
    np.testing.assert_array_equal(host(alpha_t), alpha)
    off_t = dev(off)

    def fresh():
        return (torch.full((rows, N), SENTINEL, dtype=torch.int16, device="cuda"),
                torch.full((1,), -7, dtype=torch.int32, device="cuda"))

    def done(d, st):
        assert int(host(st)[0]) == 0
        return bits(d)

    say("moe workload: grouped GEMM, [E][N][K/2] weights")
    d, st = fresh()
    nv.nvfp4_grouped_gemm(qa_t, sfa_t, b_t, bsf_t, off_t, alpha_t, d, rows, N, K, E, None, st)
    outs = {"plain": (done(d, st), 0)}
    pb, psf = nv.grouped_pack(b_t, bsf_t, N, K, E)
    del b_t, bsf_t
    say("moe workload: grouped GEMM, packed weights")
    d, st = fresh()
    nv.nvfp4_grouped_gemm_packed(qa_t, sfa_t, pb, psf, off_t, alpha_t, d, rows, N, K, E, st)
    outs["packed"] = (done(d, st), 0)
    say("moe workload: fused quantisation, packed weights")
    d, st = fresh()
    nv.nvfp4_grouped_gemm_packed_fused(dev(xb.view(np.int16)), tok_t.to(torch.int32), gsa_t, pb, psf, off_t,
                                       alpha_t, d, rows, T, N, K, E, st)
    outs["packed_fused"] = (done(d, st), 1)
    # the unfused GPU sequence on the same bf16 tokens gives the same bits
    xq_t, xsf_t = gpu_quantize(dev(o.bf16_bits_to_f32(xb)), gsa_t)
    d, st = fresh()
    nv.nvfp4_grouped_gemm_packed(xq_t[tok_t].contiguous(), xsf_t[tok_t].contiguous(), pb, psf, off_t, alpha_t, d,
                                 rows, N, K, E, st)
    np.testing.assert_array_equal(done(d, st), outs["packed_fused"][0])
    for name, (db, aset) in outs.items():
        assert not (db == SENTINEL).any(), name
        total = op.Stats()
        for e in range(E):
            lo, hi = int(off[e]), int(off[e + 1])
            if hi > lo:
                s, ref, tol = oracle_rows[e][aset]
                total.add(op.compare(db[lo:hi], s, tol, ref).check(f"{name} expert {e}", strict_frac=None))
        total.check(name)
        assert total.n == rows * N
        say(f"{name}: {total.n} elements, frob {total.frob:.3g}, strict 2-ulp {total.strict / total.n:.6f}")
    np.testing.assert_array_equal(outs["plain"][0], outs["packed"][0])
