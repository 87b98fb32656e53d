"""GPU quantiser, tensor scale and alpha: bit-exact parity with the oracle."""
import numpy as np
import pytest
import torch

import synth
from oracle import nvfp4_ref as o
from tests import oracle_pool as op
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


def test_e2m1_rounding_exhaustive_up_to_six():
    # every fp32 bit pattern of magnitude <= 6 in both signs (2 x 1,086,324,737
    # values, -0, subnormals and 6 itself included), 15 to a block behind an
    # anchor of 6: the block scale is 1 (0x38) and r = 1, so each code must be
    # the oracle's e2m1 code of the value itself.  Larger magnitudes cannot
    # keep r = 1 (they raise the block amax); the scale tests cover them.
    top = int(np.float32(6.0).view(np.uint32)) + 1
    chunk = 1 << 24
    jobs = [(lo, min(lo + chunk, top), neg) for neg in (False, True) for lo in range(0, top, chunk)]
    done = 0
    with op.make_pool() as pool:
        for i, ((lo, hi, neg), want) in enumerate(zip(jobs, pool.imap(op.e2m1_codes_of_patterns, jobs))):
            if i % 16 == 0:
                say("e2m1 exhaustive", f"chunk {i} of {len(jobs)}", "negative" if neg else "positive", hex(lo))
            vals = synth.fp32_bit_patterns(lo, hi, neg)
            n = len(vals)
            nb = -(-n // 15)
            body = np.zeros(nb * 15, np.float32)
            body[:n] = vals
            blk = np.empty((nb, 16), np.float32)
            blk[:, 0] = 6.0
            blk[:, 1:] = body.reshape(nb, 15)
            q_t, sf_t = gpu_quantize(dev(blk), None)
            sf, q = host(sf_t), host(q_t)
            assert (sf == 0x38).all(), f"patterns {hex(lo)}..{hex(hi)}: a block scale is not 1"
            codes = np.empty((nb, 16), np.uint8)
            codes[:, 0::2] = q & 0xF
            codes[:, 1::2] = q >> 4
            assert (codes[:, 0] == 0x7).all()
            got = codes[:, 1:].reshape(-1)[:n]
            if not np.array_equal(got, want):
                j = int(np.flatnonzero(got != want)[0])
                raise AssertionError(f"e2m1 code of fp32 pattern {int(vals[j:j + 1].view(np.uint32)[0]):#010x} "
                                     f"({vals[j]!r}): GPU {got[j]:#x}, oracle {want[j]:#x}")
            done += n
    assert done == 2 * top


def _e4m3_midpoints() -> np.ndarray:
    """Every midpoint between consecutive non-negative finite e4m3 values
    (codes 0x00..0x7E), plus the one above 448 that saturation removes."""
    v = np.array([o.e4m3_value(c) for c in range(0x7F)], np.float64)
    mids = np.concatenate([(v[:-1] + v[1:]) / 2, [464.0]])
    assert (mids.astype(np.float32).astype(np.float64) == mids).all()   # exact in fp32
    return mids.astype(np.float32)


def test_e4m3_scale_ties_and_subnormal_seam():
    # t = (amax / 6) * gs lands exactly on every e4m3 midpoint (the scale
    # rounds to the even code), with its fp32 neighbours on either side.
    # 1) gs = 1, block amax = 6 * mid: 6 * mid is exact and so is (6 * mid) / 6.
    mids = _e4m3_midpoints()
    seam = np.float32(2.0 ** -6 - 2.0 ** -10)        # between 7 * 2^-9 (0x07) and 2^-6 (0x08)
    assert seam in mids
    ts = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9))])
    rng = np.random.default_rng(12)
    blocks = np.zeros((len(ts), 16), np.float32)
    blocks[:, 0] = np.float32(6.0) * ts
    blocks[:, 1:] = (rng.uniform(-1, 1, (len(ts), 15)) * blocks[:, :1]).astype(np.float32)
    flat = np.concatenate([blocks.reshape(-1), np.zeros((-blocks.size) % 64, np.float32)])
    x = flat.reshape(-1, 64)
    _check_quant(x, np.float32(1), None, "e4m3 ties, gs = 1")
    # the oracle's scale bytes at the exact midpoints are the even codes
    _, sf = o.quantize(blocks[: len(mids)], np.float32(1))
    lo = np.array([c for c in range(0x7E)] + [0x7E])
    even = np.where(lo % 2 == 0, lo, lo + 1)
    even[-1] = 0x7E                                       # 464 saturates to 448
    np.testing.assert_array_equal(sf[:, 0], even)
    # 2) block amax = 6 and gs = the midpoint itself, for the seam and a few
    # subnormal, normal and top midpoints (one tensor scale per call)
    for gs in [seam, mids[0], mids[3], mids[40], mids[100], mids[-2], mids[-1]]:
        blk = np.zeros((4, 64), np.float32)
        blk[:, ::16] = 6.0
        blk[:, 1::16] = -6.0 * np.float32(0.3)
        blk[:, 5::16] = np.float32(2.9)
        gs_t = torch.tensor([gs], dtype=torch.float32, device="cuda")
        _check_quant(blk, np.float32(gs), gs_t, f"e4m3 tie gs = {float(gs)!r}")
