"""GPU quantiser, tensor scale and alpha: bit-exact parity with the oracle."""
import numpy as np
import pytest
import torch

import synth
from oracle import nvfp4_ref as o
from tests.gpu_util import dev, gpu_global_scale, gpu_quantize, host, say

pytestmark = pytest.mark.gpu


def _check_quant(x, gs_np, gs_t, label):
    say("quantize", label, x.shape)
    q_ref, sf_ref = o.quantize(x, gs_np)
    q, sf = gpu_quantize(dev(x), gs_t)
    np.testing.assert_array_equal(host(sf), sf_ref, err_msg=f"{label}: scales")
    np.testing.assert_array_equal(host(q), q_ref, err_msg=f"{label}: codes")


def test_smoke_shapes_unit_global_scale():
    a, b = synth.single_operands("smoke_128x256x256")
    _check_quant(a, np.float32(1), None, "smoke A")
    _check_quant(b, np.float32(1), None, "smoke B")


@pytest.mark.parametrize("name", ["attn_proj_n768_k6144", "moe_expert_n2048_k6144"])
def test_workload_tensors_with_global_scale(name):
    a, b = synth.single_operands(name)
    for x, lab in ((a, "A"), (b, "B")):
        xt = dev(x)
        say("global scale", name, lab)
        gs_t = gpu_global_scale(xt)
        gs_ref = o.global_encode_scale(x)
        assert host(gs_t)[0] == gs_ref, (host(gs_t)[0], gs_ref)
        _check_quant(x, gs_ref, gs_t, f"{name} {lab}")


def test_large_activation_sampled_rows():
    # 16384 x 6144 activations: global scale over the whole tensor, codes
    # compared on a seeded sample of rows (rows are independent given gs)
    a, _ = synth.single_operands("large_n6144_k6144", 16384)
    at = dev(a)
    say("global scale large A")
    gs_t = gpu_global_scale(at)
    gs_ref = o.global_encode_scale(a)
    assert host(gs_t)[0] == gs_ref
    say("quantize large A")
    q, sf = gpu_quantize(at, gs_t)
    rows = np.unique(np.concatenate([np.random.default_rng(0).choice(16384, 384, replace=False), [0, 16383]]))
    q_ref, sf_ref = o.quantize(a[rows], gs_ref)
    np.testing.assert_array_equal(host(sf[torch.from_numpy(rows).to(sf.device)]), sf_ref)
    np.testing.assert_array_equal(host(q[torch.from_numpy(rows).to(q.device)]), q_ref)


def test_rounding_ties_and_edges():
    # blocks with amax exactly 6 and gs = 1 (scale 1, r = 1) carrying every
    # e2m1 tie and its fp32 neighbours; zero blocks; -0; saturation
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    vals = np.concatenate([ties, np.nextafter(ties, 0), np.nextafter(ties, 10), -ties, [0.0, -0.0, 6.0, -6.0]])
    vals = vals.astype(np.float32)
    rows = []
    for i in range(0, len(vals), 15):
        blk = np.zeros(16, np.float32)
        blk[0] = 6.0
        part = vals[i:i + 15]
        blk[1:1 + len(part)] = part
        rows.append(blk)
    x = np.concatenate(rows)
    x = np.concatenate([x, np.zeros(16, np.float32), np.full(16, -0.0, np.float32),
                        np.full(16, 1e30, np.float32)])
    x = np.concatenate([x, np.zeros((-len(x)) % 64, np.float32)]).reshape(-1, 64)
    _check_quant(x, np.float32(1), None, "ties")


@pytest.mark.parametrize("gs", [1.0, 0.001, 3000.0])
def test_wide_dynamic_range(gs):
    # magnitudes from 2^-40 to 2^40 exercise subnormal scales, rounding up into
    # the normal range, and saturation at 448
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((256, 512)) * np.exp2(rng.uniform(-40, 40, (256, 1)))).astype(np.float32)
    gs_t = torch.tensor([gs], dtype=torch.float32, device="cuda")
    _check_quant(x, np.float32(gs), gs_t, f"wide gs={gs}")


def test_alpha_from_scales():
    import nvfp4_block_scaled_07_amd as nv
    rng = np.random.default_rng(8)
    gs_a = np.float32(rng.uniform(1, 5000))
    gs_b = rng.uniform(1e3, 1e6, 256).astype(np.float32)
    al = torch.empty(256, dtype=torch.float32, device="cuda")
    say("alpha")
    nv.nvfp4_alpha_from_scales(dev(np.array([gs_a], np.float32)), dev(gs_b), al, 256)
    want = np.array([o.alpha_from_scales(gs_a, g) for g in gs_b], np.float32)
    np.testing.assert_array_equal(host(al), want)


def test_all_zero_tensor_scale_is_one():
    x = torch.zeros(1000, dtype=torch.float32, device="cuda")
    say("zero tensor scale")
    assert host(gpu_global_scale(x))[0] == np.float32(1.0)
