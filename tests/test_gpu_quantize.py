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


def _anchored_blocks(vals: np.ndarray, anchor: float) -> np.ndarray:
    """Blocks of 16 whose first element is `anchor` (|anchor| = 6 sets the
    block scale to exactly 1 at gs = 1, so r = 1 and the codes are e2m1(x))
    and whose other 15 elements are `vals` (|v| <= 6), as rows of 64."""
    n = -(-len(vals) // 15)
    blk = np.zeros((n, 16), np.float32)
    blk[:, 0] = anchor
    body = np.zeros(n * 15, np.float32)
    body[:len(vals)] = vals
    blk[:, 1:] = body.reshape(n, 15)
    flat = blk.reshape(-1)
    flat = np.concatenate([flat, np.zeros((-len(flat)) % 64, np.float32)])
    return flat.reshape(-1, 64)


def test_e2m1_rounding_sweep_over_fp32_patterns():
    # every 61st fp32 bit pattern in [0, 6] (about 17.8 million values) plus a
    # dense window of +-2048 patterns around each rounding threshold, in both
    # signs: the GPU's e2m1 rounding must give the oracle's codes everywhere
    hi = int(np.float32(6.0).view(np.uint32))
    bits = np.arange(0, hi + 1, 61, dtype=np.uint32)
    windows = [np.arange(int(np.float32(t).view(np.uint32)) - 2048, int(np.float32(t).view(np.uint32)) + 2049,
                         dtype=np.uint32) for t in (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0)]
    bits = np.concatenate([bits, np.arange(0, 4096, dtype=np.uint32)] + windows)
    vals = bits.view(np.float32)
    vals = vals[np.abs(vals) <= 6.0]
    for sign, anchor in ((1.0, 6.0), (-1.0, -6.0)):
        x = _anchored_blocks((vals * np.float32(sign)).astype(np.float32), anchor)
        for lo in range(0, x.shape[0], 1 << 16):
            part = np.ascontiguousarray(x[lo:lo + (1 << 16)])
            _check_quant(part, np.float32(1), None, f"e2m1 sweep sign {sign:+.0f} rows {lo}")
