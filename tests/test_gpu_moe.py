"""GPU parity of the MoE expert FFN pieces through the C ABI: the SwiGLU
quantiser (codes and scales equal to the oracle's wherever they are unique),
the combine (at its fp32 summation bound), and nvfp4_moe_ffn (bit for bit
equal to the same steps called one by one, and within 1e-2 relative
Frobenius error of the oracle).  At the pages' shape every stage is compared
element by element: each GEMM with the oracle fed the stage's own inputs."""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_07_amd as nv
import synth
from oracle import moe_ref as m
from oracle import nvfp4_ref as o
from tests import oracle_pool as op
from tests.gpu_util import bits, check_gemm, dev, host, say, scalar

pytestmark = pytest.mark.gpu


def _bf16(x32):
    return torch.from_numpy(np.ascontiguousarray(x32, np.float32)).to(torch.bfloat16).view(torch.int16).numpy() \
        .view(np.uint16)


def _check_swiglu_codes(q, sf, gu_bits, I, gs):
    """Blocks whose codes are unique (the same under a 2^-20 relative change
    of h either way) must match exactly; the others must match one of the
    three quantisations, element by element."""
    rq, rsf = m.swiglu_quantize(gu_bits, I, gs)
    (lq, lsf), (hq, hsf) = m.swiglu_quantize_bounds(gu_bits, I, gs)
    rows = gu_bits.shape[0]
    codes = lambda qq: np.stack([qq & 0xF, qq >> 4], axis=-1).reshape(rows, I // 16, 16)
    c, rc, lc, hc = codes(q), codes(rq), codes(lq), codes(hq)
    unique = (rsf == lsf) & (rsf == hsf) & (rc == lc).all(-1) & (rc == hc).all(-1)
    assert (sf[unique] == rsf[unique]).all(), "scale differs on a unique block"
    assert (c[unique] == rc[unique]).all(), "codes differ on a unique block"
    amb = ~unique
    ok_sf = (sf == rsf) | (sf == lsf) | (sf == hsf)
    ok_c = (c == rc) | (c == lc) | (c == hc)
    assert ok_sf[amb].all() and ok_c[amb].all(), "an ambiguous block matches none of the admissible results"
    return int(amb.sum()), unique.size


def test_swiglu_quantize_parity():
    rng = np.random.default_rng(21)
    rows, I = 333, 1040
    g = (rng.standard_normal((rows, I)) * 4).astype(np.float32)
    g[0, :16] = -120.0          # silu underflows: a zero block
    g[1, :16] = 90.0            # silu(g) = g
    u = rng.standard_normal((rows, I)).astype(np.float32)
    gu = _bf16(np.concatenate([g, u], axis=1))
    h_amax = np.abs(m.swiglu(gu, I)).max()
    gs = np.float32(2688.0) / np.float32(h_amax)
    q = torch.empty((rows, I // 2), dtype=torch.uint8, device="cuda")
    sf = torch.empty((rows, I // 16), dtype=torch.uint8, device="cuda")
    say("swiglu quantize", rows, I)
    nv.nvfp4_swiglu_quantize(dev(gu.view(np.int16)), rows, I, scalar(gs), q, sf)
    amb, n = _check_swiglu_codes(host(q), host(sf), gu, I, gs)
    say("ambiguous blocks", amb, "of", n)
    assert amb <= n // 100


def test_combine_parity():
    rng = np.random.default_rng(22)
    T, H, k, rows = 77, 1032, 8, 616
    down = _bf16((rng.standard_normal((rows, H)) * 3).astype(np.float32))
    rows_of = rng.integers(0, rows, (T, k)).astype(np.int32)
    rows_of[3, 2] = -1
    rows_of[5, 7] = rows + 3
    w = rng.uniform(-1, 1, (T, k)).astype(np.float32)
    out = torch.empty((T, H), dtype=torch.int16, device="cuda")
    say("combine", T, H, k)
    nv.nvfp4_moe_combine(dev(down.view(np.int16)), dev(rows_of), dev(w), out, T, H, k, rows)
    got = o.bf16_to_f64(bits(out))
    ref = m.moe_combine(down, rows_of, w)
    tol = m.combine_tolerance(down, rows_of, w, ref)
    assert (np.abs(got - o.bf16_to_f64(ref)) <= tol).all()


def _ffn_problem(T, H, I, E, k, seed):
    tok, off = synth.routing(seed, T, E, k)
    tok = tok.astype(np.int32)
    tr = synth.token_rows(tok, T, k)
    tw = synth.routing_weights(seed + 1, T, k)
    x = _bf16(synth.token_activations(T, H))
    w_gu = synth.random_codes(seed + 2, E * 2 * I, H).reshape(E, 2 * I, H // 2)
    w_gu_sf = synth.random_scale_bytes(seed + 3, E * 2 * I, H, lo=0x28, hi=0x38).reshape(E, 2 * I, H // 16)
    w_d = synth.random_codes(seed + 4, E * H, I).reshape(E, H, I // 2)
    w_d_sf = synth.random_scale_bytes(seed + 5, E * H, I, lo=0x28, hi=0x38).reshape(E, H, I // 16)
    x32 = o.bf16_bits_to_f32(x)
    gs_x = o.global_encode_scale(x32)
    # scales calibrated on the first expert's rows with the oracle: gate/up
    # outputs of rms 2, h scaled to half the e4m3 x e2m1 range, down of rms 1
    e0 = int(np.argmax(np.diff(off) > 0))
    rr = tok[off[e0]:off[e0 + 1]]
    qa, sfa = o.quantize(x32[rr], gs_x)
    s_gu = o.gemm_fp64(qa, sfa, w_gu[e0], w_gu_sf[e0])
    a_gu = np.full(E, 2.0 / np.sqrt(np.mean(s_gu ** 2)), np.float32)
    h = m.swiglu(o.bf16_rne(s_gu * np.float64(a_gu[0])), I)
    gs_h = np.float32(2688.0 / (2.0 * np.abs(h).max()))
    hq, hsf = o.quantize(h.astype(np.float32), gs_h)
    s_d = o.gemm_fp64(hq, hsf, w_d[e0], w_d_sf[e0])
    a_d = np.full(E, 1.0 / np.sqrt(np.mean(s_d ** 2)), np.float32)
    return dict(tok=tok, off=off, tr=tr, tw=tw, x=x, w_gu=w_gu, w_gu_sf=w_gu_sf, w_d=w_d, w_d_sf=w_d_sf,
                gs_x=gs_x, a_gu=a_gu, gs_h=gs_h, a_d=a_d)


def _run_ffn(P, T, H, I, E, k):
    t = {n: dev(v) for n, v in P.items() if isinstance(v, np.ndarray) and n not in ("w_gu", "w_gu_sf", "w_d", "w_d_sf", "x")}
    t["x"] = dev(P["x"].view(np.int16))
    pgu, pgusf = nv.grouped_pack(dev(P["w_gu"]), dev(P["w_gu_sf"]), 2 * I, H, E)
    pd, pdsf = nv.grouped_pack(dev(P["w_d"]), dev(P["w_d_sf"]), H, I, E)
    gs_x, gs_h = scalar(P["gs_x"]), scalar(P["gs_h"])
    ws = torch.empty(nv.nvfp4_moe_ffn_workspace_size(T, H, I, k), dtype=torch.uint8, device="cuda")
    out = torch.empty((T, H), dtype=torch.int16, device="cuda")
    st = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    nv.nvfp4_moe_ffn(t["x"], gs_x, t["tok"], t["off"], pgu, pgusf, t["a_gu"], gs_h, pd, pdsf, t["a_d"], t["tr"],
                     t["tw"], out, T, H, I, E, k, ws, st)
    assert int(host(st)[0]) == 0
    # the same steps called one by one
    rows = T * k
    gu = torch.empty((rows, 2 * I), dtype=torch.int16, device="cuda")
    nv.nvfp4_grouped_gemm_packed_fused(t["x"], t["tok"], gs_x, pgu, pgusf, t["off"], t["a_gu"], gu, rows, T, 2 * I,
                                       H, E)
    hq = torch.empty((rows, I // 2), dtype=torch.uint8, device="cuda")
    hsf = torch.empty((rows, I // 16), dtype=torch.uint8, device="cuda")
    nv.nvfp4_swiglu_quantize(gu, rows, I, gs_h, hq, hsf)
    down = torch.empty((rows, H), dtype=torch.int16, device="cuda")
    nv.nvfp4_grouped_gemm_packed(hq, hsf, pd, pdsf, t["off"], t["a_d"], down, rows, H, I, E)
    out2 = torch.empty((T, H), dtype=torch.int16, device="cuda")
    nv.nvfp4_moe_combine(down, t["tr"], t["tw"], out2, T, H, k, rows)
    np.testing.assert_array_equal(bits(out), bits(out2))
    return bits(out), bits(gu)


def _frob(got_bits, ref_bits):
    g, r = o.bf16_to_f64(got_bits), o.bf16_to_f64(ref_bits)
    return np.linalg.norm(g - r) / np.linalg.norm(r)


def test_moe_ffn_small_against_oracle():
    T, H, I, E, k = 64, 1024, 512, 8, 4
    P = _ffn_problem(T, H, I, E, k, seed=300)
    say("moe ffn small", T, H, I, E, k)
    out, gu = _run_ffn(P, T, H, I, E, k)
    ref, _ = m.moe_ffn(P["x"], P["gs_x"], P["tok"], P["off"], P["w_gu"], P["w_gu_sf"], P["a_gu"], P["gs_h"],
                       P["w_d"], P["w_d_sf"], P["a_d"], P["tr"], P["tw"], I)
    # the gate/up GEMM at the GEMM tolerance, per expert
    x32 = o.bf16_bits_to_f32(P["x"])
    qa, sfa = o.quantize(o.gather_rows(x32, P["tok"], T * k), P["gs_x"])
    for e in range(E):
        lo, hi = int(P["off"][e]), int(P["off"][e + 1])
        if hi > lo:
            check_gemm(gu[lo:hi], qa[lo:hi], sfa[lo:hi], P["w_gu"][e], P["w_gu_sf"][e], P["a_gu"][e], f"gu {e}")
    fr = _frob(out, ref)
    say("ffn relative Frobenius error", fr)
    assert fr <= 1e-2


@pytest.mark.timeout(1200)
def test_moe_ffn_pages_shape_every_token():
    # the pages' layer: 512 tokens, top-8 of 256 experts, H = 6144, I = 2048,
    # each expert's weights seeded on their own.  Every element of every
    # stage is checked: gate/up against the oracle at the GEMM tolerance, the
    # SwiGLU codes where unique, down against the oracle fed with the GPU's own
    # h, the combine at its summation bound, and the layer end to end against
    # the pure-oracle chain (relative Frobenius error).
    T, H, I, E, k, seed = 512, 6144, 2048, 256, 8, 400
    rows = T * k
    tok, off = synth.routing(seed, T, E, k)
    tok = tok.astype(np.int32)
    tr = synth.token_rows(tok, T, k)
    tw = synth.routing_weights(seed + 1, T, k)
    x = _bf16(synth.token_activations(T, H))
    x32 = o.bf16_bits_to_f32(x)
    gs_x = o.global_encode_scale(x32)
    say("moe ffn 512 tokens: weights")
    w_gu = torch.empty((E, 2 * I, H // 2), dtype=torch.uint8, device="cuda")
    w_gu_sf = torch.empty((E, 2 * I, H // 16), dtype=torch.uint8, device="cuda")
    w_d = torch.empty((E, H, I // 2), dtype=torch.uint8, device="cuda")
    w_d_sf = torch.empty((E, H, I // 16), dtype=torch.uint8, device="cuda")
    for e in range(E):
        for t, v in zip((w_gu, w_gu_sf, w_d, w_d_sf), op.ffn_expert_weights(seed, e, H, I)):
            t[e].copy_(torch.from_numpy(v))
    # scales calibrated with the oracle on the first expert's rows, as in _ffn_problem
    qa, sfa = o.quantize(o.gather_rows(x32, tok, rows), gs_x)
    e0 = int(np.argmax(np.diff(off) > 0))
    wg0, wgs0, wd0, wds0 = op.ffn_expert_weights(seed, e0, H, I)
    s_gu = o.gemm_fp64(qa[off[e0]:off[e0 + 1]], sfa[off[e0]:off[e0 + 1]], wg0, wgs0)
    a_gu = np.full(E, 2.0 / np.sqrt(np.mean(s_gu ** 2)), np.float32)
    h = m.swiglu(o.bf16_rne(s_gu * np.float64(a_gu[0])), I)
    gs_h = np.float32(2688.0 / (2.0 * np.abs(h).max()))
    hq0, hsf0 = o.quantize(h.astype(np.float32), gs_h)
    s_d = o.gemm_fp64(hq0, hsf0, wd0, wds0)
    a_d = np.full(E, 1.0 / np.sqrt(np.mean(s_d ** 2)), np.float32)

    say("moe ffn 512 tokens: run")
    pgu, pgusf = nv.grouped_pack(w_gu, w_gu_sf, 2 * I, H, E)
    pd, pdsf = nv.grouped_pack(w_d, w_d_sf, H, I, E)
    del w_gu, w_gu_sf, w_d, w_d_sf
    x_t, tok_t, off_t, tr_t, tw_t = dev(x.view(np.int16)), dev(tok), dev(off), dev(tr), dev(tw)
    gs_x_t, gs_h_t, a_gu_t, a_d_t = scalar(gs_x), scalar(gs_h), dev(a_gu), dev(a_d)
    ws = torch.empty(nv.nvfp4_moe_ffn_workspace_size(T, H, I, k), dtype=torch.uint8, device="cuda")
    out = torch.empty((T, H), dtype=torch.int16, device="cuda")
    st = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    nv.nvfp4_moe_ffn(x_t, gs_x_t, tok_t, off_t, pgu, pgusf, a_gu_t, gs_h_t, pd, pdsf, a_d_t, tr_t, tw_t, out,
                     T, H, I, E, k, ws, st)
    assert int(host(st)[0]) == 0
    # the same steps one by one, for their intermediates
    gu = torch.empty((rows, 2 * I), dtype=torch.int16, device="cuda")
    nv.nvfp4_grouped_gemm_packed_fused(x_t, tok_t, gs_x_t, pgu, pgusf, off_t, a_gu_t, gu, rows, T, 2 * I, H, E)
    hq = torch.empty((rows, I // 2), dtype=torch.uint8, device="cuda")
    hsf = torch.empty((rows, I // 16), dtype=torch.uint8, device="cuda")
    nv.nvfp4_swiglu_quantize(gu, rows, I, gs_h_t, hq, hsf)
    down = torch.empty((rows, H), dtype=torch.int16, device="cuda")
    nv.nvfp4_grouped_gemm_packed(hq, hsf, pd, pdsf, off_t, a_d_t, down, rows, H, I, E)
    out2 = torch.empty((T, H), dtype=torch.int16, device="cuda")
    nv.nvfp4_moe_combine(down, tr_t, tw_t, out2, T, H, k, rows)
    out_b, gu_b, hq_h, hsf_h, down_b = bits(out), bits(gu), host(hq), host(hsf), bits(down)
    np.testing.assert_array_equal(out_b, bits(out2))

    say("moe ffn 512 tokens: oracle, every expert")
    jobs = []
    for e in range(E):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi > lo:
            jobs.append((seed, e, H, I, qa[lo:hi], sfa[lo:hi], a_gu[e], gs_h, a_d[e], gu_b[lo:hi], hq_h[lo:hi],
                         hsf_h[lo:hi], down_b[lo:hi]))
    st_gu, st_d = op.Stats(), op.Stats()
    chain = np.zeros((rows, H), np.uint16)
    with op.make_pool() as pool:
        for e, sg, sd, ch in pool.imap(op.ffn_expert_oracle, jobs):
            st_gu.add(sg.check(f"gate/up expert {e}", strict_frac=None))
            st_d.add(sd.check(f"down expert {e}", strict_frac=None))
            chain[int(off[e]):int(off[e + 1])] = ch
    st_gu.check("gate/up")
    st_d.check("down (GPU h)")
    assert st_gu.n == rows * 2 * I and st_d.n == rows * H
    say("gate/up", st_gu.n, "elements, frob", st_gu.frob, "; down", st_d.n, "elements, frob", st_d.frob)
    amb, n = _check_swiglu_codes(hq_h, hsf_h, gu_b, I, gs_h)
    say("swiglu: ambiguous blocks", amb, "of", n)
    assert amb <= n // 100
    ref = m.moe_combine(down_b, tr, tw)
    tol = m.combine_tolerance(down_b, tr, tw, ref)
    assert (np.abs(o.bf16_to_f64(out_b) - o.bf16_to_f64(ref)) <= tol).all(), "combine outside its bound"
    fr = _frob(out_b, m.moe_combine(chain, tr, tw))
    say("layer vs the pure-oracle chain: relative Frobenius error", fr)
    assert fr <= 1e-2


def test_moe_ffn_graph_replays_match_eager():
    # the whole layer (status word included) captured in one HIP graph; each
    # replay, with eager work and synchronisation in between, equals the eager run
    T, H, I, E, k = 48, 1024, 512, 6, 2
    P = _ffn_problem(T, H, I, E, k, seed=500)
    t = {n: dev(v) for n, v in P.items() if isinstance(v, np.ndarray) and n not in ("w_gu", "w_gu_sf", "w_d", "w_d_sf", "x")}
    x = dev(P["x"].view(np.int16))
    pgu, pgusf = nv.grouped_pack(dev(P["w_gu"]), dev(P["w_gu_sf"]), 2 * I, H, E)
    pd, pdsf = nv.grouped_pack(dev(P["w_d"]), dev(P["w_d_sf"]), H, I, E)
    gs_x, gs_h = scalar(P["gs_x"]), scalar(P["gs_h"])
    ws = torch.empty(nv.nvfp4_moe_ffn_workspace_size(T, H, I, k), dtype=torch.uint8, device="cuda")
    out = torch.zeros((T, H), dtype=torch.int16, device="cuda")
    st = torch.full((1,), -7, dtype=torch.int32, device="cuda")

    def run():
        nv.nvfp4_moe_ffn(x, gs_x, t["tok"], t["off"], pgu, pgusf, t["a_gu"], gs_h, pd, pdsf, t["a_d"], t["tr"],
                         t["tw"], out, T, H, I, E, k, ws, st)
    say("ffn graph eager")
    run()
    eager = bits(out).copy()
    assert int(host(st)[0]) == 0
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        run()
    for rep in range(3):
        out.fill_(0)
        ws.fill_(0xFF)
        st.fill_(-7)
        torch.cuda.synchronize()
        say("ffn graph replay", rep)
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bits(out), eager)
        assert int(host(st)[0]) == 0


def test_moe_ffn_single_token_and_empty_experts():
    # one token routed to 2 of 5 experts: three experts have no rows
    T, H, I, E, k = 1, 512, 512, 5, 2
    P = _ffn_problem(T, H, I, E, k, seed=600)
    assert (np.diff(P["off"]) == 0).sum() == 3
    say("moe ffn single token")
    out, _ = _run_ffn(P, T, H, I, E, k)
    ref, _ = m.moe_ffn(P["x"], P["gs_x"], P["tok"], P["off"], P["w_gu"], P["w_gu_sf"], P["a_gu"], P["gs_h"],
                       P["w_d"], P["w_d_sf"], P["a_d"], P["tr"], P["tw"], I)
    assert _frob(out, ref) <= 1e-2


def test_moe_ffn_tall_experts():
    # 128 tokens, top-2 of 4 experts: about 64 rows per expert, so both
    # grouped GEMMs take their 64-row passes
    T, H, I, E, k = 128, 512, 1024, 4, 2
    P = _ffn_problem(T, H, I, E, k, seed=700)
    assert T * k > 40 * E
    say("moe ffn tall experts", np.diff(P["off"]))
    out, _ = _run_ffn(P, T, H, I, E, k)
    ref, _ = m.moe_ffn(P["x"], P["gs_x"], P["tok"], P["off"], P["w_gu"], P["w_gu_sf"], P["a_gu"], P["gs_h"],
                       P["w_d"], P["w_d_sf"], P["a_d"], P["tr"], P["tw"], I)
    fr = _frob(out, ref)
    say("ffn relative Frobenius error", fr)
    assert fr <= 1e-2
