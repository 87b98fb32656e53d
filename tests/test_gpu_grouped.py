"""GPU grouped-by-expert GEMM parity with the oracle: adversarial row
distributions, every grouped kernel, invalid offsets and the packed weight
layout (the 512-token, 256-expert workload itself, every expert, is in
test_gpu_moe_workload.py)."""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_07_amd as nv
import synth
from oracle import nvfp4_ref as o
from tests.gpu_util import bits, check_gemm, dev, host, say

pytestmark = pytest.mark.gpu
SENTINEL = 0x7FC1


def _grouped(a_t, asf_t, b_t, bsf_t, off_t, alpha_t, rows, N, K, E, status=True):
    d = torch.full((max(rows, 1), max(N, 1)), SENTINEL, dtype=torch.int16, device="cuda")
    st = torch.full((1,), -7, dtype=torch.int32, device="cuda") if status else None
    need = nv.nvfp4_grouped_workspace_size(rows, N, K, E)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda") if need else None
    nv.nvfp4_grouped_gemm(a_t, asf_t, b_t, bsf_t, off_t, alpha_t, d, rows, N, K, E, ws, st)
    return d, st


def _small_problem(kind, rows=300, E=8, N=192, K=512, seed=0):
    off = synth.adversarial_offsets(kind, rows, E) if isinstance(kind, str) else np.asarray(kind, np.int32)
    a = synth.random_codes(seed + 1, rows, K)
    asf = synth.random_scale_bytes(seed + 2, rows, K, lo=0x30, hi=0x40)
    b = synth.random_codes(seed + 3, E * N, K).reshape(E, N, K // 2)
    bsf = synth.random_scale_bytes(seed + 4, E * N, K, lo=0x30, hi=0x40).reshape(E, N, K // 16)
    alpha = np.linspace(0.5, 2.0, E).astype(np.float32)
    return off, a, asf, b, bsf, alpha


@pytest.mark.parametrize("kind", ["one", "alternate", "ones", "empty",
                                  [0, 0, 5, 5, 70, 70, 71, 200, 250], [0, 16, 32, 48, 64, 80, 96, 112, 128]])
def test_adversarial_row_distributions(kind):
    rows, E, N, K = 300, 8, 192, 512
    off, a, asf, b, bsf, alpha = _small_problem(kind, rows, E, N, K)
    say("grouped adversarial", kind)
    d, st = _grouped(dev(a), dev(asf), dev(b), dev(bsf), dev(off), dev(alpha), rows, N, K, E)
    assert int(host(st)[0]) == 0
    want = o.grouped_gemm(a, asf, b, bsf, off, alpha, np.full((rows, N), SENTINEL, np.uint16))
    db = bits(d)
    for e in range(E):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi > lo:
            check_gemm(db[lo:hi], a[lo:hi], asf[lo:hi], b[e], bsf[e], alpha[e], f"{kind} expert {e}")
    # rows beyond offsets[E] are untouched
    np.testing.assert_array_equal(db[int(off[-1]):], want[int(off[-1]):])


def test_null_alpha_and_no_status():
    off, a, asf, b, bsf, _ = _small_problem([0, 40, 41, 100, 100, 160, 161, 162, 300])
    say("grouped null alpha")
    d, _ = _grouped(dev(a), dev(asf), dev(b), dev(bsf), dev(off), None, 300, 192, 512, 8, status=False)
    db = bits(d)
    for e in range(8):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi > lo:
            check_gemm(db[lo:hi], a[lo:hi], asf[lo:hi], b[e], bsf[e], np.float32(1), f"expert {e}")


def test_invalid_offsets_reported_and_skipped():
    # expert 3's range decreases: status = 1 + 3; other experts still computed
    off = np.array([0, 10, 20, 60, 50, 70, 80, 90, 100], np.int32)
    _, a, asf, b, bsf, alpha = _small_problem("empty")
    say("grouped invalid offsets")
    d, st = _grouped(dev(a), dev(asf), dev(b), dev(bsf), dev(off), dev(alpha), 300, 192, 512, 8)
    assert int(host(st)[0]) == 4
    db = bits(d)
    # expert 4's range [50, 70) overlaps expert 2's [20, 60): check the rows
    # that only one valid expert writes
    for e, lo, hi in ((0, 0, 10), (1, 10, 20), (2, 20, 50), (4, 60, 70), (5, 70, 80), (6, 80, 90), (7, 90, 100)):
        check_gemm(db[lo:hi], a[lo:hi], asf[lo:hi], b[e], bsf[e], alpha[e], f"expert {e}")
    # offsets beyond rows: status names the first such expert
    off2 = np.array([0, 10, 20, 30, 40, 50, 60, 70, 400], np.int32)
    d2, st2 = _grouped(dev(a), dev(asf), dev(b), dev(bsf), dev(off2), dev(alpha), 300, 192, 512, 8)
    assert int(host(st2)[0]) == 8
    assert (bits(d2)[70:] == SENTINEL).all()


@pytest.mark.parametrize("gplan,K", [(0, 768), (1, 768), (2, 1536), (2, 768), (3, 1024), (3, 1536), (3, 768)])
def test_every_grouped_kernel(gplan, K, force_plan):
    # each grouped kernel (forced through nvfp4_force_plan; K = 1536 lets the
    # register kernels' prefetch depth 2 divide K / 256, K = 768 does not and
    # must fall back), ragged N, experts of 0, 1, 5, 65 and 129 rows (several
    # row passes of 32 or 64 rows)
    force_plan(nv.FAMILY_GROUPED, gplan)
    rows, E, N = 300, 8, 330
    off, a, asf, b, bsf, alpha = _small_problem([0, 0, 5, 5, 70, 70, 71, 200, 250], rows, E, N, K, seed=40)
    say("grouped kernel", gplan, "K", K)
    d, st = _grouped(dev(a), dev(asf), dev(b), dev(bsf), dev(off), dev(alpha), rows, N, K, E)
    assert int(host(st)[0]) == 0
    db = bits(d)
    for e in range(E):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi > lo:
            check_gemm(db[lo:hi], a[lo:hi], asf[lo:hi], b[e], bsf[e], alpha[e], f"gplan {gplan} expert {e}")
    assert (db[250:] == SENTINEL).all()


def _np_pack(b, bsf, N, K, E):
    """Reference of the packed weight layout (numpy rearrangement)."""
    T, n = -(-N // 256), K // 256
    bp = np.zeros((E, T * 256, K // 2), np.uint8)
    bp[:, :N] = b
    sp = np.zeros((E, T * 256, K // 16), np.uint8)
    sp[:, :N] = bsf
    blocks = bp.reshape(E, T, 256, n, 8, 16).transpose(0, 1, 3, 2, 4, 5)  # [E][T][n][row][chunk][16 B]
    # inside a block, 16-byte chunk c of row r goes to position
    # (((r // 32) * 2 + (r % 32) // 16) * 2 + c // 4) * 64 + (c % 4) * 16 + r % 16
    r, c = np.meshgrid(np.arange(256), np.arange(8), indexing="ij")
    pos = (((r // 32) * 2 + (r % 32) // 16) * 2 + c // 4) * 64 + (c % 4) * 16 + r % 16
    out = np.zeros((E, T, n, 2048, 16), np.uint8)
    out[:, :, :, pos.reshape(-1), :] = blocks.reshape(E, T, n, 2048, 16)
    # blocks in stage-major order: stage, then expert, then slab
    pb = np.ascontiguousarray(out.transpose(2, 0, 1, 3, 4)).reshape(-1)
    # scale block: word w (bytes 4w .. 4w+3) of row r goes to word position
    # ((((r // 32) * 16 + r % 16) * 2 + w % 2) * 4 + ((r % 32) // 16) * 2 + w // 2
    words = np.ascontiguousarray(sp.reshape(E, T, 256, n, 16).transpose(0, 1, 3, 2, 4)).view(np.uint32)
    words = words.reshape(E, T, n, 256, 4)
    r, w = np.meshgrid(np.arange(256), np.arange(4), indexing="ij")
    wpos = (((r // 32) * 16 + r % 16) * 2 + w % 2) * 4 + ((r % 32) // 16) * 2 + w // 2
    sf = np.zeros((E, T, n, 1024), np.uint32)
    sf[:, :, :, wpos.reshape(-1)] = words.reshape(E, T, n, 1024)
    psf = np.ascontiguousarray(sf.transpose(2, 0, 1, 3)).view(np.uint8).reshape(-1)
    return pb, psf


@pytest.mark.parametrize("gplan", [2, 3])
@pytest.mark.parametrize("kind", ["alternate", [0, 0, 5, 5, 70, 70, 71, 200, 250]])
def test_packed_weights_layout_and_gemm(kind, gplan, force_plan):
    # gplan 2 / 3: passes of 32 / 64 rows over each expert's packed weights
    force_plan(nv.FAMILY_GROUPED, gplan)
    rows, E, N, K = 300, 8, 330, 1024
    off, a, asf, b, bsf, alpha = _small_problem(kind, rows, E, N, K, seed=60)
    say("grouped packed", kind, "gplan", gplan)
    b_t, bsf_t = dev(b), dev(bsf)
    pb, psf = nv.grouped_pack(b_t, bsf_t, N, K, E)
    want_pb, want_psf = _np_pack(b, bsf, N, K, E)
    np.testing.assert_array_equal(host(pb), want_pb)
    np.testing.assert_array_equal(host(psf), want_psf)
    d = torch.full((rows, N), SENTINEL, dtype=torch.int16, device="cuda")
    st = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    nv.nvfp4_grouped_gemm_packed(dev(a), dev(asf), pb, psf, dev(off), dev(alpha), d, rows, N, K, E, st)
    assert int(host(st)[0]) == 0
    db = bits(d)
    for e in range(E):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi > lo:
            check_gemm(db[lo:hi], a[lo:hi], asf[lo:hi], b[e], bsf[e], alpha[e], f"packed {kind} expert {e}")
    assert (db[int(off[-1]):] == SENTINEL).all()
    # same bits as the unpacked grouped kernel (same arithmetic, same order)
    d2, _ = _grouped(dev(a), dev(asf), b_t, bsf_t, dev(off), dev(alpha), rows, N, K, E)
    np.testing.assert_array_equal(bits(d2), db)


# nvfp4_grouped_gemm_sf: activation and weight scales in a tiled layout (the
# weights' scales as one [E * N][K/16] matrix), read in place.  N = 300 puts
# experts at rows that are not multiples of 8 or 128 of that matrix.
@pytest.mark.parametrize("layout", [1, 2])
@pytest.mark.parametrize("gplan", [-1, 2, 3])
@pytest.mark.parametrize("kind,N,K", [("alternate", 300, 1024), ([0, 0, 5, 5, 70, 70, 71, 200, 250], 192, 512),
                                      ([0, 40, 90, 150, 200, 250, 251, 252, 300], 256, 1536),
                                      ("ones", 130, 512)])
def test_grouped_gemm_on_tiled_scales(layout, gplan, kind, N, K, force_plan):
    # gplan: the automatic kernel, or the 32-row (2) or 64-row (3) register kernel forced
    rows, E = 300, 8
    force_plan(nv.FAMILY_GROUPED, gplan)
    off, a, asf, b, bsf, alpha = _small_problem(kind, rows, E, N, K, seed=N + K)
    to = o.scales_to_128x4 if layout == 1 else o.scales_to_8x4
    a_t, b_t, off_t, al_t = dev(a), dev(b), dev(off), dev(alpha)
    say("grouped tiled scales", layout, kind, N, K)
    d = torch.full((rows, N), SENTINEL, dtype=torch.int16, device="cuda")
    st = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    nv.nvfp4_grouped_gemm_sf(a_t, dev(to(asf)), b_t, dev(to(bsf.reshape(E * N, K // 16))), off_t, al_t, d,
                             rows, N, K, E, layout, st)
    assert int(host(st)[0]) == 0
    ref, _ = _grouped(a_t, dev(asf), b_t, dev(bsf), off_t, al_t, rows, N, K, E)
    np.testing.assert_array_equal(bits(d), bits(ref))
    db = bits(d)
    for e in range(E):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi > lo:
            check_gemm(db[lo:hi], a[lo:hi], asf[lo:hi], b[e], bsf[e], alpha[e], f"tiled {layout} expert {e}")
    assert (db[int(off[-1]):] == SENTINEL).all()
