"""GPU GEMM parity with the oracle through the C ABI, at every plan the
library picks for the page workloads, plus ragged, degenerate and invariant
cases."""
import json
import os

import numpy as np
import pytest
import torch

import nvfp4_block_scaled_07_amd as nv
import synth
from oracle import nvfp4_ref as o
from tests.gpu_util import bits, check_gemm, dev, gpu_gemm, gpu_global_scale, gpu_quantize, host, say, scalar

pytestmark = pytest.mark.gpu
GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _quantized_workload(name, m=None):
    """oracle-side and GPU-side quantisation of the same seeded fp32 inputs;
    the bytes must agree before the GEMM is compared."""
    a, b = synth.single_operands(name, m)
    w = synth.WORKLOADS[name]
    at, bt = dev(a), dev(b)
    if w["unit_global_scale"]:
        gsa = gsb = np.float32(1)
        gsa_t = gsb_t = None
        alpha = np.float32(1)
        alpha_t = scalar(1.0)
    else:
        gsa, gsb = o.global_encode_scale(a), o.global_encode_scale(b)
        gsa_t, gsb_t = gpu_global_scale(at), gpu_global_scale(bt)
        alpha = o.alpha_from_scales(gsa, gsb)
        alpha_t = torch.empty(1, dtype=torch.float32, device="cuda")
        nv.nvfp4_alpha_from_scales(gsa_t, gsb_t, alpha_t, 1)
        assert host(alpha_t)[0] == alpha
    qa, sfa = o.quantize(a, gsa)
    qb, sfb = o.quantize(b, gsb)
    qa_t, sfa_t = gpu_quantize(at, gsa_t)
    qb_t, sfb_t = gpu_quantize(bt, gsb_t)
    np.testing.assert_array_equal(host(qa_t), qa)
    np.testing.assert_array_equal(host(sfa_t), sfa)
    np.testing.assert_array_equal(host(qb_t), qb)
    np.testing.assert_array_equal(host(sfb_t), sfb)
    return (qa, sfa, qb, sfb, alpha), (qa_t, sfa_t, qb_t, sfb_t, alpha_t)


def test_worked_fixture_padded_to_k256():
    with open(os.path.join(GOLD, "worked_gemm_2x3x32.json")) as f:
        g = json.load(f)
    rows = lambda hexes, per: np.frombuffer(b"".join(bytes.fromhex(h) for h in hexes), np.uint8).reshape(-1, per)
    pad = lambda x, w: np.concatenate([x, np.zeros((x.shape[0], w - x.shape[1]), np.uint8)], axis=1)
    a = pad(rows(g["a_hex"], 16), 128)
    asf = pad(rows(g["a_sf_hex"], 2), 16)
    b = pad(rows(g["b_hex"], 16), 128)
    bsf = pad(rows(g["b_sf_hex"], 2), 16)
    say("worked fixture")
    d = gpu_gemm(dev(a), dev(asf), dev(b), dev(bsf), scalar(1.0), 2, 3, 256)
    np.testing.assert_array_equal(o.bf16_to_f64(bits(d)), np.array(g["expected"]))
    d = gpu_gemm(dev(a), dev(asf), dev(b), dev(bsf), scalar(0.5), 2, 3, 256)
    np.testing.assert_array_equal(o.bf16_to_f64(bits(d)), np.array(g["alpha_half_expected"]))
    d = gpu_gemm(dev(a), dev(asf), dev(b), dev(bsf), None, 2, 3, 256)   # NULL alpha = 1
    np.testing.assert_array_equal(o.bf16_to_f64(bits(d)), np.array(g["expected"]))


def test_smoke_workload_not_all_zeros_and_matches():
    ref, gpu = _quantized_workload("smoke_128x256x256")
    say("smoke gemm 128x256x256")
    d = gpu_gemm(*gpu, 128, 256, 256)
    db = bits(d)
    v = o.bf16_to_f64(db)
    assert not (v == 0).all() and np.isfinite(v).all()
    check_gemm(db, *ref, label="smoke")


def test_random_bytes_like_the_page_smoke_test():
    # the pages' kernel test fed random code bytes and random scale bytes
    M, N, K = 128, 256, 256
    a, b = synth.random_codes(11, M, K), synth.random_codes(12, N, K)
    asf, bsf = synth.random_scale_bytes(13, M, K), synth.random_scale_bytes(14, N, K)
    say("random bytes 128x256x256")
    d = gpu_gemm(dev(a), dev(asf), dev(b), dev(bsf), scalar(1.0), M, N, K)
    st = check_gemm(bits(d), a, asf, b, bsf, np.float32(1), "random bytes")
    assert st["n"] == M * N


@pytest.mark.parametrize("name", ["attn_proj_n768_k6144", "moe_expert_n2048_k6144", "decode_wide_n16384_k6144"])
def test_decode_and_prefill_sweeps(name):
    w = synth.WORKLOADS[name]
    ref, gpu = _quantized_workload(name)
    qa, sfa, qb, sfb, alpha = ref
    for m in w["ms"]:
        say(name, "M =", m, "plan", nv.nvfp4_gemm_plan(m, w["n"], w["k"]))
        d = gpu_gemm(gpu[0][:m], gpu[1][:m], gpu[2], gpu[3], gpu[4], m, w["n"], w["k"])
        st = check_gemm(bits(d), qa[:m], sfa[:m], qb, sfb, alpha, f"{name} M={m}")
        assert st["strict_2ulp_frac"] > 0.999


@pytest.mark.parametrize("M,N,K", [(1, 1, 256), (17, 129, 512), (100, 200, 768), (65, 96, 256),
                                   (129, 130, 1024), (33, 5, 2048), (300, 1000, 256),
                                   # automatic split plans on ragged tiles whose K stages do not
                                   # divide evenly over the splits (K-group tile split five ways
                                   # over 10 and 25 stages; register tiles split two ways)
                                   (300, 500, 2560), (130, 1000, 6400), (20, 900, 2048),
                                   # wide weights at decode M (32x32 register tiles, unsplit)
                                   (24, 9000, 512)])
def test_ragged_shapes(M, N, K):
    a, b = synth.random_codes(M * 7 + 1, M, K), synth.random_codes(N * 7 + 2, N, K)
    asf = synth.random_scale_bytes(M + 3, M, K, lo=0x28, hi=0x48, signed=True)
    bsf = synth.random_scale_bytes(N + 4, N, K, lo=0x28, hi=0x48)
    say("ragged", M, N, K, nv.nvfp4_gemm_plan(M, N, K))
    d = gpu_gemm(dev(a), dev(asf), dev(b), dev(bsf), scalar(0.75), M, N, K, d_fill=0x7FC1)
    check_gemm(bits(d), a, asf, b, bsf, np.float32(0.75), f"ragged {M}x{N}x{K}")


def test_deterministic_and_sign_flip():
    for (M, N, K) in [(16, 768, 6144), (300, 384, 1024), (512, 512, 2048), (2048, 2048, 256)]:
        a, b = synth.random_codes(1, M, K), synth.random_codes(2, N, K)
        asf = synth.random_scale_bytes(3, M, K, lo=0x30, hi=0x40)
        bsf = synth.random_scale_bytes(4, N, K, lo=0x30, hi=0x40)
        at, asft, bt, bsft = dev(a), dev(asf), dev(b), dev(bsf)
        say("determinism", M, N, K, nv.nvfp4_gemm_plan(M, N, K))
        d1 = bits(gpu_gemm(at, asft, bt, bsft, scalar(1.0), M, N, K))
        d2 = bits(gpu_gemm(at, asft, bt, bsft, scalar(1.0), M, N, K))
        np.testing.assert_array_equal(d1, d2)
        dn = bits(gpu_gemm(dev(a ^ np.uint8(0x88)), asft, bt, bsft, scalar(1.0), M, N, K))
        np.testing.assert_array_equal(o.bf16_to_f64(dn), -o.bf16_to_f64(d1))


def test_zero_sized_calls_are_noops():
    d = torch.full((4, 4), 7, dtype=torch.int16, device="cuda")
    x = torch.zeros((4, 128), dtype=torch.uint8, device="cuda")
    s = torch.zeros((4, 16), dtype=torch.uint8, device="cuda")
    say("zero sized")
    nv.nvfp4_gemm(x, s, x, s, None, d, 0, 4, 256)
    nv.nvfp4_gemm(x, s, x, s, None, d, 4, 0, 256)
    assert (host(d) == 7).all()


def test_split_k_workspace_reuse_and_counters_return_to_zero(force_plan):
    # one workspace, zero-filled once, serves several split-K shapes in a row
    # (auto plans: the K-group and register tiles, and the skinny split-K
    # tile forced for M = 16 and 64);
    # afterwards every arrival counter is back at zero
    shapes = [(16, 768, 6144, "3"), (1024, 256, 6144, None), (64, 2048, 6144, "4"), (300, 384, 1024, "11,3"),
              (16, 768, 6144, None), (32, 768, 6144, "10,2"), (16, 768, 6144, "3")]
    need = 0
    for (M, N, K, forced) in shapes:
        force_plan(nv.FAMILY_GEMM, *map(int, forced.split(","))) if forced else force_plan(nv.FAMILY_GEMM, -1)
        assert nv.nvfp4_gemm_workspace_size(M, N, K) > 0, (M, N, K)
        need = max(need, nv.nvfp4_gemm_workspace_size(M, N, K))
    ws = nv.nvfp4_workspace_init(torch.empty(need, dtype=torch.uint8, device="cuda"))
    for (M, N, K, forced) in shapes:
        force_plan(nv.FAMILY_GEMM, *map(int, forced.split(","))) if forced else force_plan(nv.FAMILY_GEMM, -1)
        a, b = synth.random_codes(M, M, K), synth.random_codes(N, N, K)
        asf = synth.random_scale_bytes(M + 1, M, K, lo=0x30, hi=0x40)
        bsf = synth.random_scale_bytes(N + 1, N, K, lo=0x30, hi=0x40)
        d = torch.empty((M, N), dtype=torch.int16, device="cuda")
        say("workspace reuse", M, N, K, nv.nvfp4_gemm_plan(M, N, K))
        nv.nvfp4_gemm(dev(a), dev(asf), dev(b), dev(bsf), None, d, M, N, K, ws)
        check_gemm(bits(d), a, asf, b, bsf, np.float32(1), f"reuse {M}x{N}x{K}")
        # the arrival counters occupy the first 4096 bytes of every split-K
        # workspace; a completed call leaves all of them at zero
        counters = host(ws)[:4096].view(np.int32)
        assert (counters == 0).all(), counters


def test_graph_capture_replays_match_eager():
    # register K-group (M = 16 splits K in two), split-K K-group (M = 1024,
    # N = 256) and single-pass plans captured in one HIP graph; each replay,
    # with eager work and synchronisation in between, must equal the eager run
    cases = [(16, 768, 6144), (512, 768, 6144), (1024, 256, 6144), (256, 768, 6144), (2048, 2048, 512)]
    ins, outs, eager = [], [], []
    for (M, N, K) in cases:
        a, b = synth.random_codes(M + 5, M, K), synth.random_codes(N + 5, N, K)
        asf = synth.random_scale_bytes(M + 6, M, K, lo=0x30, hi=0x40)
        bsf = synth.random_scale_bytes(N + 6, N, K, lo=0x30, hi=0x40)
        t = (dev(a), dev(asf), dev(b), dev(bsf), nv.gemm_workspace(M, N, K))
        ins.append(t)
        d = torch.zeros((M, N), dtype=torch.int16, device="cuda")
        outs.append(d)
        say("graph eager", M, N, K, nv.nvfp4_gemm_plan(M, N, K))
        nv.nvfp4_gemm(t[0], t[1], t[2], t[3], None, d, M, N, K, t[4])
        eager.append(bits(d).copy())
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    say("graph capture")
    with torch.cuda.graph(g):
        for (M, N, K), t, d in zip(cases, ins, outs):
            nv.nvfp4_gemm(t[0], t[1], t[2], t[3], None, d, M, N, K, t[4])
    for rep in range(3):
        for d in outs:
            d.fill_(0)
        torch.cuda.synchronize()
        say("graph replay", rep)
        g.replay()
        torch.cuda.synchronize()
        for d, e in zip(outs, eager):
            np.testing.assert_array_equal(bits(d), e)


def test_every_plan_kind_forced(force_plan):
    # each kernel instantiation (plan kind), with and without split-K, on a
    # ragged shape; the plan is forced through nvfp4_force_plan(kind, splits)
    M, N, K = 200, 330, 1536
    a, b = synth.random_codes(91, M, K), synth.random_codes(92, N, K)
    asf = synth.random_scale_bytes(93, M, K, lo=0x28, hi=0x48)
    bsf = synth.random_scale_bytes(94, N, K, lo=0x28, hi=0x48)
    at, asft, bt, bsft = dev(a), dev(asf), dev(b), dev(bsf)
    seen = set()
    for kind in range(24):  # past the last kind the plan falls back to auto (deduplicated)
        for splits in (1, 3):
            force_plan(nv.FAMILY_GEMM, kind, splits)
            plan = nv.nvfp4_gemm_plan(M, N, K)
            if plan in seen and splits == 1:
                continue
            seen.add(plan)
            say("forced plan", kind, splits, plan, nv.nvfp4_gemm_workspace_size(M, N, K))
            d = gpu_gemm(at, asft, bt, bsft, scalar(1.25), M, N, K, d_fill=0x7FC1)
            check_gemm(bits(d), a, asf, b, bsf, np.float32(1.25), f"plan {plan} splits {splits}")
            # bitwise deterministic: a second call (fresh workspace) repeats every bit
            d2 = gpu_gemm(at, asft, bt, bsft, scalar(1.25), M, N, K, d_fill=0x1234)
            np.testing.assert_array_equal(bits(d2), bits(d), err_msg=f"plan {plan} splits {splits} rerun")
    force_plan(nv.FAMILY_GEMM, -1)
    assert len(seen) >= 6


@pytest.mark.parametrize("M,N,K", [(40, 200, 1536), (16, 768, 6144), (1, 17, 256)])
def test_register_tiles_split_k_forced(force_plan, M, N, K):
    # the register-streamed tiles (128- and 256-element K units) with split-K
    # forced on ragged shapes: partial rows and columns, K of one unit
    a, b = synth.random_codes(M + 101, M, K), synth.random_codes(N + 102, N, K)
    asf = synth.random_scale_bytes(103, M, K, lo=0x28, hi=0x48)
    bsf = synth.random_scale_bytes(104, N, K, lo=0x28, hi=0x48)
    at, asft, bt, bsft = dev(a), dev(asf), dev(b), dev(bsf)
    seen = set()
    for kind in range(10, 16):   # past the last kind the plan falls back to auto
        for splits in (1, 2, 3):
            force_plan(nv.FAMILY_GEMM, kind, splits)
            key = (nv.nvfp4_gemm_plan(M, N, K), nv.nvfp4_gemm_workspace_size(M, N, K))
            if not key[0].startswith("kreg") or key in seen:
                continue
            seen.add(key)
            say("register tile", M, N, K, kind, splits, key)
            d = gpu_gemm(at, asft, bt, bsft, scalar(0.5), M, N, K, d_fill=0x7FC1)
            check_gemm(bits(d), a, asf, b, bsf, np.float32(0.5), f"{key} splits {splits}")
    force_plan(nv.FAMILY_GEMM, -1)
    assert len(seen) >= (4 if K == 256 else 11)


def test_maximum_k_every_plan_kind(force_plan):
    # K = 2^22, the largest supported K: a row of codes is 2 MB, so a 256-row
    # operand tile spans 512 MB of 32-bit buffer offsets.  Every plan kind
    # (split-K forced to 3 where it applies) on a ragged 17 x 24 output,
    # against one oracle evaluation.
    M, N, K = 17, 24, 1 << 22
    a, b = synth.random_codes(131, M, K), synth.random_codes(132, N, K)
    asf = synth.random_scale_bytes(133, M, K, lo=0x30, hi=0x40)
    bsf = synth.random_scale_bytes(134, N, K, lo=0x30, hi=0x40)
    alpha = np.float32(2.0 ** -6)
    say("max K oracle")
    s = o.gemm_fp64(a, asf, b, bsf) * np.float64(alpha)
    ref = o.bf16_rne(s)
    tol = o.gemm_tolerance(a, asf, b, bsf, alpha, ref)
    want = o.bf16_to_f64(ref)
    at, asft, bt, bsft = dev(a), dev(asf), dev(b), dev(bsf)
    seen = set()
    for kind in range(24):
        for splits in (1, 3):
            force_plan(nv.FAMILY_GEMM, kind, splits)
            key = (nv.nvfp4_gemm_plan(M, N, K), nv.nvfp4_gemm_workspace_size(M, N, K))
            if key in seen:
                continue
            seen.add(key)
            say("max K plan", kind, splits, key)
            d = gpu_gemm(at, asft, bt, bsft, scalar(alpha), M, N, K, d_fill=0x7FC1)
            got = o.bf16_to_f64(bits(d))
            assert (np.abs(got - want) <= tol).all(), f"{key}: outside tolerance"
            assert np.linalg.norm(got - s) / np.linalg.norm(s) <= 1e-2, key
    force_plan(nv.FAMILY_GEMM, -1)
    assert len(seen) >= 10
