"""CPU checks of the process-pool helpers the full-output GPU tests use: a
block comparison accepts the oracle's own output and rejects a planted
error, the per-expert helpers return the oracle's bytes, and the
statistics add up over blocks."""
import numpy as np

import synth
from oracle import moe_ref as m
from oracle import nvfp4_ref as o
from tests import oracle_pool as op


def _problem(M=96, N=40, K=512):
    a, b = synth.random_codes(1, M, K), synth.random_codes(2, N, K)
    asf = synth.random_scale_bytes(3, M, K, lo=0x30, hi=0x40)
    bsf = synth.random_scale_bytes(4, N, K, lo=0x30, hi=0x40)
    return a, asf, b, bsf


def test_block_comparison_in_the_pool():
    a, asf, b, bsf = _problem()
    alpha = np.float32(0.75)
    want = o.gemm(a, asf, b, bsf, alpha)
    bad = want.copy()
    bad[70, 3] ^= np.uint16(0x40)                  # mantissa bit 6 flipped, in the second block
    jobs = [("nv", a[r:r + 48], asf[r:r + 48], b, bsf, alpha, [want[r:r + 48], bad[r:r + 48]]) for r in (0, 48)]
    with op.make_pool(2) as pool:
        res = pool.map(op.gemm_rows_compare, jobs)
    good, wrong = op.Stats(), op.Stats()
    for r in res:
        good.add(r[0])
        wrong.add(r[1])
    good.check("oracle against itself")
    assert good.n == 96 * 40 and good.bad == 0 and good.strict == good.n and good.frob < 1e-2
    assert wrong.n == good.n and wrong.bad == 1


def test_expert_helper_returns_the_oracle_bytes():
    e, n, k = 5, 32, 512
    qa, sfa = o.quantize(synth.token_activations(3, k), np.float32(20.0))
    got = op.expert_oracle((e, np.float32(20.0), [(qa, sfa)], n, k))
    w = synth.expert_weights(e, n, k)
    gs = o.global_encode_scale(w)
    qb, sfb = o.quantize(w, gs)
    assert got[0] == e and got[3] == gs and got[4] == o.alpha_from_scales(np.float32(20.0), gs)
    np.testing.assert_array_equal(got[1], qb)
    np.testing.assert_array_equal(got[2], sfb)
    s, ref, tol = got[5][0]
    np.testing.assert_array_equal(ref, o.gemm(qa, sfa, qb, sfb, got[4]))
    assert (tol > 0).all()


def test_ffn_helper_matches_the_layer_oracle():
    seed, e, H, I = 900, 2, 512, 512
    w_gu, w_gu_sf, w_d, w_d_sf = op.ffn_expert_weights(seed, e, H, I)
    x = synth.token_activations(4, H)
    qa, sfa = o.quantize(x, np.float32(50.0))
    a_gu, gs_h, a_d = np.float32(0.01), np.float32(300.0), np.float32(0.02)
    gu = o.gemm(qa, sfa, w_gu, w_gu_sf, a_gu)
    hq, hsf = m.swiglu_quantize(gu, I, gs_h)
    down = o.gemm(hq, hsf, w_d, w_d_sf, a_d)
    e_, st_gu, st_d, chain = op.ffn_expert_oracle((seed, e, H, I, qa, sfa, a_gu, gs_h, a_d, gu, hq, hsf, down))
    assert e_ == e and st_gu.bad == 0 and st_d.bad == 0 and st_gu.n == 4 * 2 * I and st_d.n == 4 * H
    np.testing.assert_array_equal(chain, down)


def test_e2m1_sweep_helpers():
    # the pattern generator gives the fp32 values of consecutive bit patterns,
    # and the pool helper returns the oracle's codes of exactly those values
    six = int(np.float32(6.0).view(np.uint32))
    v = synth.fp32_bit_patterns(six - 2, six + 2)
    assert v[2] == np.float32(6.0) and v[1] == np.nextafter(np.float32(6.0), np.float32(0))
    neg = synth.fp32_bit_patterns(0, 3, negative=True)
    assert np.signbit(neg).all() and neg[0] == 0 and neg[1] == -np.float32(2.0 ** -149)
    lo, hi = int(np.float32(0.2).view(np.uint32)), int(np.float32(0.3).view(np.uint32))
    for negative in (False, True):
        got = op.e2m1_codes_of_patterns((lo, hi, negative))
        np.testing.assert_array_equal(got, o.e2m1_encode(synth.fp32_bit_patterns(lo, hi, negative)))
        quarter = int(np.float32(0.25).view(np.uint32)) - lo      # the 0 / 0.5 tie rounds to 0
        sign = 0x8 if negative else 0
        assert got[quarter] == sign and got[quarter + 1] == (sign | 1) and got[quarter - 1] == sign
