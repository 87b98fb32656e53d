"""The C ABI loads and exports every declared symbol; host-side validation
returns the documented status codes.  CPU only: every call below is rejected
(or answered) on the host before any HIP call, so no GPU is needed."""
import ctypes
import os
import re

import pytest

import nvfp4_block_scaled_07_amd as nv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(nvfp4_\w+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    names = _declared()
    assert "nvfp4_gemm" in names and "nvfp4_grouped_gemm" in names
    lib = nv.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(nv.SIGNATURES), "binding and header disagree"


def test_binding_loads_in_tree_library():
    assert os.path.dirname(nv.LIB_PATH) == os.path.join(ROOT, "nvfp4_block_scaled_07_amd")
    maps = open("/proc/self/maps").read()
    nv.lib()
    assert nv.LIB_PATH in open("/proc/self/maps").read() or nv.LIB_PATH in maps


FAKE = 0x10000  # an aligned non-NULL address; never dereferenced (calls are rejected on the host)


def _gemm(a=FAKE, asf=FAKE, b=FAKE, bsf=FAKE, alpha=None, d=FAKE, M=16, N=16, K=256, ws=None, wsb=0):
    return nv.lib().nvfp4_gemm(a, asf, b, bsf, alpha, d, M, N, K, ws, wsb, None)


def test_gemm_error_paths():
    assert _gemm(K=40) == 2 and "block size 16" in nv.nvfp4_last_error()
    assert _gemm(K=-16) == 2
    assert _gemm(M=-1) == 2
    assert _gemm(K=128) == 4 and "256" in nv.nvfp4_last_error()
    assert _gemm(K=0) == 4
    assert _gemm(K=(1 << 22) + 256) == 4 and "4194304" in nv.nvfp4_last_error()
    assert nv.nvfp4_gemm_workspace_size(16, 768, (1 << 22) + 256) == 0
    assert _gemm(a=None) == 1
    assert _gemm(d=None) == 1
    assert _gemm(a=FAKE + 8) == 3
    assert _gemm(bsf=FAKE + 4) == 3
    assert _gemm(d=FAKE + 2) == 3
    # a split-K plan (M = 1024, N = 256: 64 K-group tiles of 64x64 split in
    # five) needs a workspace
    need = nv.nvfp4_gemm_workspace_size(1024, 256, 6144)
    assert need > 0
    assert _gemm(M=1024, N=256, K=6144) == 5 and "workspace" in nv.nvfp4_last_error()
    assert _gemm(M=1024, N=256, K=6144, ws=FAKE, wsb=need - 1) == 5
    assert _gemm(M=1024, N=256, K=6144, ws=FAKE + 16, wsb=need) == 3
    # empty problems succeed without touching anything
    assert _gemm(M=0, a=None, d=None) == 0
    assert _gemm(N=0) == 0


def test_grouped_error_paths():
    L = nv.lib()
    call = lambda **k: L.nvfp4_grouped_gemm(k.get("a", FAKE), FAKE, FAKE, FAKE, k.get("off", FAKE), None,
                                            k.get("d", FAKE), k.get("rows", 64), k.get("N", 64),
                                            k.get("K", 256), k.get("E", 4), None, 0, k.get("st", None), None)
    assert call(K=24) == 2
    assert call(E=-1) == 2
    assert call(off=None) == 1
    assert call(a=None) == 1
    assert call(off=FAKE + 2) == 3
    assert call(st=FAKE + 1) == 3
    assert call(K=384) == 4


def test_quantize_and_scale_error_paths():
    L = nv.lib()
    assert L.nvfp4_quantize(FAKE, 4, 24, None, FAKE, FAKE, None) == 2
    assert L.nvfp4_quantize(None, 4, 32, None, FAKE, FAKE, None) == 1
    assert L.nvfp4_quantize(FAKE + 4, 4, 32, None, FAKE, FAKE, None) == 3
    assert L.nvfp4_quantize(FAKE, 4, 32, None, FAKE + 4, FAKE, None) == 3  # codes 8-byte aligned
    assert L.nvfp4_quantize(None, 0, 32, None, None, None, None) == 0
    assert L.nvfp4_global_scale(FAKE, -1, FAKE, None) == 2
    assert L.nvfp4_global_scale(FAKE, 10, None, None) == 1
    assert L.nvfp4_alpha_from_scales(FAKE, FAKE, None, 3, None) == 1
    assert L.nvfp4_alpha_from_scales(None, None, None, 0, None) == 0


def test_plan_and_workspace_queries():
    assert nv.nvfp4_gemm_plan(16384, 6144, 6144).startswith("tile")
    assert nv.nvfp4_gemm_plan(16, 768, 6144).startswith("kreg16x16")
    assert nv.nvfp4_gemm_plan(64, 2048, 6144).startswith("kreg32x16")
    assert nv.nvfp4_gemm_plan(1024, 768, 6144).startswith("tile64x64k4")
    assert nv.nvfp4_gemm_workspace_size(64, 768, 6144) == 0  # 192 register tiles: no split, no workspace
    # 48 register tiles of 16x16 split K two ways: counters + fp32 partial tiles
    assert nv.nvfp4_gemm_workspace_size(16, 768, 6144) == 4096 + 48 * 2 * 16 * 16 * 4
    # above M = 128 the K-group tile, split about three work-groups per CU
    assert nv.nvfp4_gemm_plan(256, 2048, 6144).startswith("tile64x64k4")
    assert nv.nvfp4_gemm_plan(512, 768, 6144).startswith("tile64x64k4")
    assert nv.nvfp4_gemm_workspace_size(512, 768, 6144) == 4096 + 96 * 5 * 64 * 64 * 4
    assert nv.nvfp4_gemm_workspace_size(1024, 768, 6144) == 4096 + 192 * 4 * 64 * 64 * 4
    assert nv.nvfp4_gemm_plan(512, 2048, 6144).startswith("tile64x64k4")
    assert nv.nvfp4_gemm_workspace_size(1024, 2048, 6144) == 0        # 512 tiles: no split
    # 96 register tiles of 16x16 split K two ways
    assert nv.nvfp4_gemm_workspace_size(32, 768, 6144) == 4096 + 96 * 2 * 16 * 16 * 4
    assert nv.nvfp4_gemm_plan(16, 768, 100) == "none"
    assert nv.nvfp4_gemm_workspace_size(16384, 6144, 6144) == 0
    # split-K plans: a 4096-byte counter block, then fp32 partial tiles
    ws = nv.nvfp4_gemm_workspace_size(1024, 256, 6144)
    tiles = (1024 // 64) * (256 // 64)
    assert ws == 4096 + tiles * 5 * 64 * 64 * 4


def test_packed_grouped_error_paths():
    L = nv.lib()
    # sizes: codes and scales of E experts padded to 256-row slabs; K % 512 required
    assert nv.nvfp4_grouped_packed_size(2048, 6144, 256) == (256 * 2048 * 3072, 256 * 2048 * 384)
    assert nv.nvfp4_grouped_packed_size(330, 1024, 8) == (8 * 512 * 512, 8 * 512 * 64)
    assert nv.nvfp4_grouped_packed_size(330, 768, 8) == (0, 0)
    pack = lambda **k: L.nvfp4_grouped_pack_b(k.get("b", FAKE), FAKE, k.get("N", 64), k.get("K", 512), k.get("E", 2),
                                              k.get("p", FAKE), FAKE, None)
    assert pack(K=768) == 4 and "512" in nv.nvfp4_last_error()
    assert pack(K=40) == 2
    assert pack(N=-1) == 2
    assert pack(b=None) == 1
    assert pack(p=FAKE + 8) == 3
    assert pack(E=0, b=None) == 0
    gemm = lambda **k: L.nvfp4_grouped_gemm_packed(FAKE, FAKE, FAKE, FAKE, k.get("off", FAKE), None, k.get("d", FAKE),
                                                   k.get("rows", 64), 64, k.get("K", 512), 4, None, None)
    assert gemm(K=256) == 4
    assert gemm(off=None) == 1
    assert gemm(d=None) == 1
    assert gemm(rows=-1) == 2


def test_mx_gemm_error_paths_and_queries():
    L = nv.lib()
    call = lambda **k: L.nvfp4_mx_gemm(k.get("a", FAKE), k.get("asf", FAKE), FAKE, FAKE, None, k.get("d", FAKE),
                                       k.get("M", 16), k.get("N", 16), k.get("K", 256), k.get("ws", None),
                                       k.get("wsb", 0), None)
    assert call(K=48) == 2 and "32" in nv.nvfp4_last_error()      # not a multiple of the MX block
    assert call(K=-32) == 2
    assert call(K=160) == 4                                         # multiple of 32, not of 256
    assert call(K=(1 << 22) + 256) == 4
    assert call(M=-1) == 2
    assert call(a=None) == 1
    assert call(d=None) == 1
    assert call(a=FAKE + 8) == 3
    assert call(asf=FAKE + 2) == 3                                  # scales need 4-byte alignment
    assert call(M=0, a=None) == 0                                   # empty: success before any check
    assert nv.nvfp4_mx_gemm_plan(16, 768, 100) == "none"
    assert nv.nvfp4_mx_gemm_plan(16384, 6144, 6144).startswith("mx256x256w8")
    assert nv.nvfp4_mx_gemm_plan(16, 768, 6144).startswith("mxreg16x16")
    assert nv.nvfp4_mx_gemm_plan(512, 768, 6144).startswith("mx64x64")
    assert nv.nvfp4_mx_gemm_plan(1024, 768, 6144).startswith("mx64x64")
    # 48 register tiles of 16x16 split K in two; 64 LDS tiles of 64x64 (M = 1024,
    # N = 256) split in four; 192 of them not at all
    assert nv.nvfp4_mx_gemm_workspace_size(16, 768, 6144) == 4096 + 48 * 2 * 16 * 16 * 4
    assert nv.nvfp4_mx_gemm_workspace_size(64, 768, 6144) == 0
    assert nv.nvfp4_mx_gemm_workspace_size(1024, 256, 6144) == 4096 + 64 * 4 * 64 * 64 * 4
    # 192 tiles of 64x64 split K three ways (about two work-groups per CU)
    assert nv.nvfp4_mx_gemm_workspace_size(1024, 768, 6144) == 4096 + 192 * 3 * 64 * 64 * 4
    assert call(M=16, N=768, K=6144) == 5 and "workspace" in nv.nvfp4_last_error()
    assert nv.nvfp4_mx_gemm_workspace_size(16384, 6144, 6144) == 0


def _fused(packed=False, x=FAKE, tok=FAKE, gs=None, b=FAKE, bsf=FAKE, off=FAKE, alpha=None, d=FAKE, rows=64,
           T=32, N=256, K=512, E=4, st=None):
    fn = nv.lib().nvfp4_grouped_gemm_packed_fused if packed else nv.lib().nvfp4_grouped_gemm_fused
    return fn(x, tok, gs, b, bsf, off, alpha, d, rows, T, N, K, E, st, None)


@pytest.mark.parametrize("packed", [False, True])
def test_fused_grouped_error_paths(packed):
    assert _fused(packed, K=256) == 4 and "512" in nv.nvfp4_last_error()
    assert _fused(packed, K=40) == 2
    assert _fused(packed, rows=-1) == 2
    assert _fused(packed, T=-1) == 2
    assert _fused(packed, T=1 << 18, K=4096) == 4 and "2^31" in nv.nvfp4_last_error()
    assert _fused(packed, tok=None, rows=64, T=32) == 2 and "row_token" in nv.nvfp4_last_error()
    assert _fused(packed, off=None) == 1
    assert _fused(packed, x=None) == 1
    assert _fused(packed, b=None) == 1
    assert _fused(packed, d=None) == 1
    assert _fused(packed, x=FAKE + 8) == 3
    assert _fused(packed, tok=FAKE + 2) == 3
    assert _fused(packed, gs=FAKE + 2) == 3
    assert _fused(packed, st=FAKE + 2) == 3
    # nothing to multiply and no status word: accepted without a launch
    assert _fused(packed, rows=0, x=None, d=None) == 0
    assert _fused(packed, E=0, off=None, x=None) == 0


def test_moe_ffn_and_pieces_error_paths():
    L = nv.lib()
    assert L.nvfp4_quantize_rows_bf16(FAKE, FAKE, None, FAKE, FAKE, 8, 4, 40, None) == 2
    assert L.nvfp4_quantize_rows_bf16(FAKE, None, None, FAKE, FAKE, 8, 4, 64, None) == 2
    assert L.nvfp4_quantize_rows_bf16(FAKE + 8, FAKE, None, FAKE, FAKE, 8, 4, 64, None) == 3
    assert L.nvfp4_quantize_rows_bf16(FAKE, FAKE, None, None, FAKE, 8, 4, 64, None) == 1
    assert L.nvfp4_swiglu_quantize(FAKE, 4, 40, None, FAKE, FAKE, None) == 2
    assert L.nvfp4_swiglu_quantize(None, 4, 64, None, FAKE, FAKE, None) == 1
    assert L.nvfp4_swiglu_quantize(FAKE + 4, 4, 64, None, FAKE, FAKE, None) == 3
    assert L.nvfp4_moe_combine(FAKE, FAKE, FAKE, FAKE, 4, 12, 2, 8, None) == 2
    assert L.nvfp4_moe_combine(FAKE, None, FAKE, FAKE, 4, 16, 2, 8, None) == 1
    assert L.nvfp4_moe_combine(FAKE + 8, FAKE, FAKE, FAKE, 4, 16, 2, 8, None) == 3
    need = L.nvfp4_moe_ffn_workspace_size(4, 512, 512, 2)
    assert need > 0

    def ffn(H=512, I=512, E=2, k=2, ws=FAKE, wsb=None, x=FAKE, T=4):
        return L.nvfp4_moe_ffn(x, None, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, None, FAKE, FAKE, FAKE,
                               T, H, I, E, k, ws, need if wsb is None else wsb, None, None)
    assert ffn(H=256) == 4 and "512" in nv.nvfp4_last_error()
    assert ffn(I=768) == 4
    assert ffn(E=0) == 2
    assert ffn(x=None) == 1
    assert ffn(ws=FAKE + 16) == 3
    assert ffn(wsb=need - 1) == 5
    assert ffn(ws=None) == 5
    assert ffn(T=0, x=None) == 0


def test_missing_library_raises_and_nothing_falls_back(monkeypatch, tmp_path):
    # the binding has no CPU path: without the built library every entry point
    # fails at load, and no module of the package imports the oracle
    monkeypatch.setattr(nv, "_lib", None)
    monkeypatch.setattr(nv, "LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(ImportError):
        nv.lib()
    with pytest.raises(ImportError):
        nv.nvfp4_gemm_plan(16, 768, 6144)
    pkg = os.path.join(ROOT, "nvfp4_block_scaled_07_amd")
    for f in os.listdir(pkg):
        if f.endswith(".py"):
            src = open(os.path.join(pkg, f)).read()
            assert "oracle" not in src.replace("no CPU or PyTorch fallback", ""), f


def test_scale_layout_error_paths_and_sizes():
    L = nv.lib()
    assert L.nvfp4_scales_128x4_size(130, 80) == 256 * 8
    assert L.nvfp4_scales_128x4_size(1, 16) == 512
    assert L.nvfp4_scales_128x4_size(4, 40) == 0
    assert L.nvfp4_scales_to_128x4(FAKE, FAKE, 4, 40, None) == 2
    assert L.nvfp4_scales_to_128x4(None, FAKE, 4, 64, None) == 1
    assert L.nvfp4_scales_from_128x4(FAKE, None, 4, 64, None) == 1
    assert L.nvfp4_scales_from_128x4(FAKE, FAKE, -1, 64, None) == 2
    assert L.nvfp4_scales_to_128x4(None, None, 0, 64, None) == 0


def test_force_plan_sets_and_restores_the_choice():
    L = nv.lib()
    auto = nv.nvfp4_gemm_plan(1024, 768, 6144)
    with nv.forced_plan(nv.FAMILY_GEMM, 0):
        assert nv.nvfp4_gemm_plan(1024, 768, 6144) == "tile256x256_mfma32"
        assert nv.nvfp4_gemm_workspace_size(1024, 768, 6144) == 0    # that kind never splits K
    assert nv.nvfp4_gemm_plan(1024, 768, 6144) == auto
    with nv.forced_plan(nv.FAMILY_GEMM, 9, 5):                          # K-group tile, 5 splits
        assert nv.nvfp4_gemm_plan(1024, 768, 6144) == "tile64x64k4_mfma32"
        assert nv.nvfp4_gemm_workspace_size(1024, 768, 6144) == 4096 + 192 * 5 * 64 * 64 * 4
    with nv.forced_plan(nv.FAMILY_GEMM, 999):                           # no such kind: own choice kept
        assert nv.nvfp4_gemm_plan(1024, 768, 6144) == auto
    auto_mx = nv.nvfp4_mx_gemm_plan(8192, 6144, 6144)
    with nv.forced_plan(nv.FAMILY_MX, 2):
        assert nv.nvfp4_mx_gemm_plan(8192, 6144, 6144) == "mx64x64_fp4mfma"
    assert nv.nvfp4_mx_gemm_plan(8192, 6144, 6144) == auto_mx
    assert L.nvfp4_force_plan(3, 0, 0) == 2 and "family" in nv.nvfp4_last_error()
    assert L.nvfp4_force_plan(-1, 0, 0) == 2
    assert L.nvfp4_force_plan(0, 1, 17) == 2
    assert nv.nvfp4_gemm_plan(1024, 768, 6144) == auto


class _FakeTensor:
    """Stands in for a torch tensor in the binding's pointer checks."""

    def __init__(self, cuda=True, contiguous=True, nbytes=1 << 20):
        self.is_cuda, self._c, self._n = cuda, contiguous, nbytes

    def is_contiguous(self):
        return self._c

    def numel(self):
        return self._n

    def element_size(self):
        return 1

    def data_ptr(self):
        return FAKE


def test_binding_rejects_host_strided_and_short_tensors():
    ok = _FakeTensor()
    M, N, K = 16, 32, 256
    d = _FakeTensor(nbytes=2 * M * N)
    for bad, status, what in ((_FakeTensor(cuda=False), 1, "GPU tensor"),
                              (_FakeTensor(contiguous=False), 2, "contiguous"),
                              (_FakeTensor(nbytes=M * K // 2 - 1), 2, "bytes")):
        with pytest.raises(nv.Nvfp4Error) as e:
            nv.nvfp4_gemm(bad, ok, ok, ok, None, d, M, N, K)
        assert e.value.status == status and what in str(e.value), str(e.value)
    with pytest.raises(nv.Nvfp4Error) as e:
        nv.nvfp4_gemm(ok, ok, ok, ok, None, _FakeTensor(nbytes=2 * M * N - 2), M, N, K)
    assert "d holds" in str(e.value)
    with pytest.raises(nv.Nvfp4Error):
        nv.nvfp4_grouped_gemm(ok, ok, ok, ok, _FakeTensor(nbytes=4 * 8), None, ok, 64, 64, 256, 8)   # offsets [E+1]
    with pytest.raises(nv.Nvfp4Error):
        nv.nvfp4_quantize(_FakeTensor(nbytes=4 * 64 * 16 - 4), 64, 16, None, ok, ok)


def test_8x4_layout_error_paths_and_sizes():
    L = nv.lib()
    assert L.nvfp4_scales_8x4_size(9, 80) == 16 * 8
    assert L.nvfp4_scales_8x4_size(1, 16) == 32
    assert L.nvfp4_scales_8x4_size(4, 40) == 0
    assert L.nvfp4_scales_to_8x4(FAKE, FAKE, 4, 40, None) == 2
    assert L.nvfp4_scales_to_8x4(None, FAKE, 4, 64, None) == 1
    assert L.nvfp4_scales_from_8x4(FAKE, None, 4, 64, None) == 1
    assert L.nvfp4_scales_from_8x4(FAKE, FAKE, -1, 64, None) == 2
    assert L.nvfp4_scales_to_8x4(None, None, 0, 64, None) == 0


def test_tiled_scale_gemm_error_paths_and_workspace():
    L = nv.lib()

    def call(layout, M=16, N=16, K=256, ws=None, wsb=0, asf=FAKE):
        return L.nvfp4_gemm_sf(FAKE, asf, FAKE, FAKE, None, FAKE, M, N, K, layout, ws, wsb, None)

    assert call(3) == 2 and "sf_layout" in nv.nvfp4_last_error()
    assert call(-1) == 2
    assert call(1, K=40) == 2 and call(2, K=128) == 4
    assert call(1, asf=None) == 1 and call(2, asf=FAKE + 4) == 3
    assert call(1, M=0) == 0
    for layout in (0, 1, 2):
        assert L.nvfp4_gemm_sf_workspace_size(16, 768, 6144, layout) == L.nvfp4_gemm_workspace_size(16, 768, 6144)
    assert L.nvfp4_gemm_sf_workspace_size(16, 768, 6144, 3) == 0
    assert L.nvfp4_gemm_sf_workspace_size(16, 768, 200, 1) == 0
    # an LDS plan reads 8 x 4 scales in place but converts 128 x 4 ones into
    # the workspace, after the plan's own split-K scratch (256-byte aligned)
    base = L.nvfp4_gemm_workspace_size(1024, 256, 6144)
    rup = lambda x: (x + 255) // 256 * 256
    need = L.nvfp4_gemm_sf_workspace_size(1024, 256, 6144, 1)
    assert need == rup(base) + rup(1024 * 384) + rup(256 * 384)
    assert call(1, M=1024, N=256, K=6144, ws=FAKE, wsb=need - 1) == 5
    assert L.nvfp4_gemm_sf_workspace_size(1024, 256, 6144, 2) == base
    assert L.nvfp4_gemm_sf_workspace_size(1024, 256, 6144, 0) == base


def test_tiled_scale_grouped_error_paths():
    L = nv.lib()

    def call(layout, rows=64, N=64, K=512, E=2, off=FAKE, asf=FAKE):
        return L.nvfp4_grouped_gemm_sf(FAKE, asf, FAKE, FAKE, off, None, FAKE, rows, N, K, E, layout, None, None)

    assert call(3) == 2 and "sf_layout" in nv.nvfp4_last_error()
    assert call(1, K=256) == 4 and "512" in nv.nvfp4_last_error()
    assert call(2, K=40) == 2
    assert call(1, off=None) == 1
    assert call(2, asf=None) == 1 and call(2, asf=FAKE + 4) == 3
    assert call(1, rows=0) == 0
