"""Python binding of the gfx950 NVFP4 library (``include/nvfp4.h``).

Argument marshalling only: every function passes device pointers, sizes and
the current HIP stream to the C ABI of ``libnvfp4_gfx950.so`` (built in-tree by
``nvfp4_block_scaled_07_amd.build``).  All arithmetic runs in the library's
HIP kernels; there is no CPU or PyTorch fallback, and a missing library is an
error.

The C entry points are exposed with their own names (``nvfp4_gemm``,
``nvfp4_grouped_gemm``, ...) taking torch tensors in place of pointers.
Tensors are used only as device memory; the stream is
``torch.cuda.current_stream()``.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libnvfp4_gfx950.so")

STATUS = {0: "NVFP4_OK", 1: "NVFP4_ERR_NULL", 2: "NVFP4_ERR_SHAPE", 3: "NVFP4_ERR_ALIGN",
          4: "NVFP4_ERR_UNSUPPORTED", 5: "NVFP4_ERR_WORKSPACE", 6: "NVFP4_ERR_HIP"}

# exported symbol -> (restype, argtypes)
_vp, _i64, _i32, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
SIGNATURES = {
    "nvfp4_gemm": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _sz, _vp]),
    "nvfp4_gemm_noalloc": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp]),
    "nvfp4_gemm_workspace_size": (_sz, [_i64, _i64, _i64]),
    "nvfp4_gemm_sf": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _vp, _sz, _vp]),
    "nvfp4_gemm_sf_workspace_size": (_sz, [_i64, _i64, _i64, _i32]),
    "nvfp4_grouped_gemm_sf": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _vp,
                                             _vp]),
    "nvfp4_workspace_init": (ctypes.c_int, [_vp, _sz, _vp]),
    "nvfp4_grouped_gemm": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _vp, _sz,
                                          _vp, _vp]),
    "nvfp4_grouped_workspace_size": (_sz, [_i64, _i64, _i64, _i32]),
    "nvfp4_grouped_packed_size": (_sz, [_i64, _i64, _i32, _vp]),
    "nvfp4_grouped_pack_b": (ctypes.c_int, [_vp, _vp, _i64, _i64, _i32, _vp, _vp, _vp]),
    "nvfp4_grouped_gemm_packed": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _vp,
                                                 _vp]),
    "nvfp4_grouped_gemm_fused": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64,
                                                _i32, _vp, _vp]),
    "nvfp4_grouped_gemm_packed_fused": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64,
                                                       _i64, _i32, _vp, _vp]),
    "nvfp4_quantize_rows_bf16": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp]),
    "nvfp4_swiglu_quantize": (ctypes.c_int, [_vp, _i64, _i64, _vp, _vp, _vp, _vp]),
    "nvfp4_moe_combine": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i32, _i64, _vp]),
    "nvfp4_moe_ffn_workspace_size": (_sz, [_i64, _i64, _i64, _i32]),
    "nvfp4_moe_ffn": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64,
                                     _i64, _i64, _i32, _i32, _vp, _sz, _vp, _vp]),
    "nvfp4_scales_128x4_size": (_sz, [_i64, _i64]),
    "nvfp4_scales_to_128x4": (ctypes.c_int, [_vp, _vp, _i64, _i64, _vp]),
    "nvfp4_scales_from_128x4": (ctypes.c_int, [_vp, _vp, _i64, _i64, _vp]),
    "nvfp4_scales_8x4_size": (_sz, [_i64, _i64]),
    "nvfp4_scales_to_8x4": (ctypes.c_int, [_vp, _vp, _i64, _i64, _vp]),
    "nvfp4_scales_from_8x4": (ctypes.c_int, [_vp, _vp, _i64, _i64, _vp]),
    "nvfp4_quantize": (ctypes.c_int, [_vp, _i64, _i64, _vp, _vp, _vp, _vp]),
    "nvfp4_global_scale": (ctypes.c_int, [_vp, _i64, _vp, _vp]),
    "nvfp4_alpha_from_scales": (ctypes.c_int, [_vp, _vp, _vp, _i32, _vp]),
    "nvfp4_gemm_plan": (ctypes.c_char_p, [_i64, _i64, _i64]),
    "nvfp4_mx_gemm": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _sz, _vp]),
    "nvfp4_mx_gemm_workspace_size": (_sz, [_i64, _i64, _i64]),
    "nvfp4_mx_gemm_plan": (ctypes.c_char_p, [_i64, _i64, _i64]),
    "nvfp4_force_plan": (ctypes.c_int, [_i32, _i32, _i32]),
    "nvfp4_last_error": (ctypes.c_char_p, []),
}

# nvfp4_force_plan families
FAMILY_GEMM, FAMILY_MX, FAMILY_GROUPED = 0, 1, 2

_lib = None


class Nvfp4Error(RuntimeError):
    def __init__(self, status: int, fn: str, msg: str):
        super().__init__(f"{fn}: {STATUS.get(status, status)}: {msg}")
        self.status = status


def lib():
    """Load the in-tree library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: run `python -m nvfp4_block_scaled_07_amd.build`")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(l, name)
            f.restype, f.argtypes = res, args
        _lib = l
    return _lib


def _ptr(t, nbytes=0, name="tensor", fn="nvfp4"):
    """Device pointer of t (None -> NULL, which the library checks itself).
    A tensor must be on the GPU, contiguous and hold at least nbytes: a host
    tensor, a strided view or a short buffer would otherwise reach a kernel
    as a wild device address."""
    if t is None:
        return None
    if not getattr(t, "is_cuda", False):
        raise Nvfp4Error(1, fn, f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise Nvfp4Error(2, fn, f"{name} must be contiguous")
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise Nvfp4Error(2, fn, f"{name} holds {have} bytes, the call needs {nbytes}")
    return ctypes.c_void_p(t.data_ptr())


def _n(*dims):
    """Product of sizes, 0 if any is negative (the library rejects those)."""
    out = 1
    for d in dims:
        if d < 0:
            return 0
        out *= d
    return out


def _bytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def _stream(stream=None):
    if stream is not None:
        return ctypes.c_void_p(stream)
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(status: int, fn: str):
    if status != 0:
        raise Nvfp4Error(status, fn, lib().nvfp4_last_error().decode())


def nvfp4_force_plan(family: int, kind: int, splits: int = 0):
    """Tuning and tests only: force the plan of a family (FAMILY_GEMM,
    FAMILY_MX, FAMILY_GROUPED) for later calls; kind < 0 restores the
    library's choice."""
    _check(lib().nvfp4_force_plan(family, kind, splits), "nvfp4_force_plan")


class forced_plan:
    """Context manager around nvfp4_force_plan that restores the library's
    own choice on exit."""

    def __init__(self, family: int, kind: int, splits: int = 0):
        self.family, self.kind, self.splits = family, kind, splits

    def __enter__(self):
        nvfp4_force_plan(self.family, self.kind, self.splits)
        return self

    def __exit__(self, *exc):
        nvfp4_force_plan(self.family, -1, 0)
        return False


def nvfp4_last_error() -> str:
    return lib().nvfp4_last_error().decode()


def nvfp4_gemm_plan(M: int, N: int, K: int) -> str:
    return lib().nvfp4_gemm_plan(M, N, K).decode()


def nvfp4_gemm_workspace_size(M: int, N: int, K: int) -> int:
    return int(lib().nvfp4_gemm_workspace_size(M, N, K))


def nvfp4_workspace_init(workspace, stream=None):
    """Zero-fill a workspace tensor (needed once before its first use)."""
    if workspace is None:
        return None
    st = lib().nvfp4_workspace_init(_ptr(workspace, 0, "workspace", "nvfp4_workspace_init"), _bytes(workspace),
                                    _stream(stream))
    _check(st, "nvfp4_workspace_init")
    return workspace


def gemm_workspace(M: int, N: int, K: int, device="cuda"):
    """Allocate and zero-fill the workspace nvfp4_gemm needs (None if none)."""
    import torch
    need = nvfp4_gemm_workspace_size(M, N, K)
    if need == 0:
        return None
    ws = torch.empty(need, dtype=torch.uint8, device=device)
    return nvfp4_workspace_init(ws)


def nvfp4_mx_gemm_plan(M: int, N: int, K: int) -> str:
    return lib().nvfp4_mx_gemm_plan(M, N, K).decode()


def nvfp4_mx_gemm_workspace_size(M: int, N: int, K: int) -> int:
    return int(lib().nvfp4_mx_gemm_workspace_size(M, N, K))


def mx_gemm_workspace(M: int, N: int, K: int, device="cuda"):
    """Allocate and zero-fill the workspace nvfp4_mx_gemm needs (None if none)."""
    import torch
    need = nvfp4_mx_gemm_workspace_size(M, N, K)
    if need == 0:
        return None
    ws = torch.empty(need, dtype=torch.uint8, device=device)
    return nvfp4_workspace_init(ws)


def nvfp4_mx_gemm(a, a_sf, b, b_sf, alpha, d, M: int, N: int, K: int, workspace=None, stream=None):
    """MXFP4 GEMM (E8M0 scales per 32 elements); see include/nvfp4.h.
    a: uint8 [M][K/2], a_sf: uint8 [M][K/32], b: uint8 [N][K/2],
    b_sf: uint8 [N][K/32], alpha: fp32 device scalar tensor or None,
    d: caller-allocated [M][N] bf16 (or int16/uint16) tensor, returned."""
    f = "nvfp4_mx_gemm"
    st = lib().nvfp4_mx_gemm(_ptr(a, _n(M, K) // 2, "a", f), _ptr(a_sf, _n(M, K) // 32, "a_sf", f),
                             _ptr(b, _n(N, K) // 2, "b", f), _ptr(b_sf, _n(N, K) // 32, "b_sf", f),
                             _ptr(alpha, 4, "alpha", f), _ptr(d, 2 * _n(M, N), "d", f), M, N, K,
                             _ptr(workspace, 0, "workspace", f), _bytes(workspace), _stream(stream))
    _check(st, "nvfp4_mx_gemm")
    return d


def nvfp4_gemm_noalloc(a, a_sf, b, b_sf, alpha, d, M: int, N: int, K: int, stream=None):
    """nvfp4_gemm without a workspace: split-K scratch in the library's fixed
    per-device array (calls overlapping on one GPU race); see include/nvfp4.h."""
    f = "nvfp4_gemm_noalloc"
    st = lib().nvfp4_gemm_noalloc(_ptr(a, _n(M, K) // 2, "a", f), _ptr(a_sf, _n(M, K) // 16, "a_sf", f),
                                  _ptr(b, _n(N, K) // 2, "b", f), _ptr(b_sf, _n(N, K) // 16, "b_sf", f),
                                  _ptr(alpha, 4, "alpha", f), _ptr(d, 2 * _n(M, N), "d", f), M, N, K,
                                  _stream(stream))
    _check(st, f)
    return d


def nvfp4_grouped_workspace_size(rows: int, N: int, K: int, E: int) -> int:
    return int(lib().nvfp4_grouped_workspace_size(rows, N, K, E))


def nvfp4_gemm(a, a_sf, b, b_sf, alpha, d, M: int, N: int, K: int, workspace=None, stream=None):
    """D = bf16(alpha * dequant(A) @ dequant(B)^T); see include/nvfp4.h.
    a: uint8 [M][K/2], a_sf: uint8 [M][K/16], b: uint8 [N][K/2],
    b_sf: uint8 [N][K/16], alpha: fp32 device scalar tensor or None,
    d: caller-allocated [M][N] bf16 (or int16/uint16) tensor, returned."""
    f = "nvfp4_gemm"
    st = lib().nvfp4_gemm(_ptr(a, _n(M, K) // 2, "a", f), _ptr(a_sf, _n(M, K) // 16, "a_sf", f),
                          _ptr(b, _n(N, K) // 2, "b", f), _ptr(b_sf, _n(N, K) // 16, "b_sf", f),
                          _ptr(alpha, 4, "alpha", f), _ptr(d, 2 * _n(M, N), "d", f), M, N, K,
                          _ptr(workspace, 0, "workspace", f), _bytes(workspace), _stream(stream))
    _check(st, "nvfp4_gemm")
    return d


# scale layouts of nvfp4_gemm_sf
SF_LINEAR, SF_128x4, SF_8x4 = 0, 1, 2


def _sf_bytes(rows: int, K: int, sf_layout: int) -> int:
    if sf_layout == SF_128x4:
        return nvfp4_scales_128x4_size(rows, K)
    if sf_layout == SF_8x4:
        return nvfp4_scales_8x4_size(rows, K)
    return _n(rows, K) // 16


def nvfp4_gemm_sf_workspace_size(M: int, N: int, K: int, sf_layout: int) -> int:
    return int(lib().nvfp4_gemm_sf_workspace_size(M, N, K, sf_layout))


def nvfp4_gemm_sf(a, a_sf, b, b_sf, alpha, d, M: int, N: int, K: int, sf_layout: int, workspace=None,
                  stream=None):
    """nvfp4_gemm with a_sf and b_sf in the scale layout sf_layout (SF_128x4,
    SF_8x4 or SF_LINEAR, tiled bytes as nvfp4_scales_to_128x4 / _8x4 write
    them); see include/nvfp4.h.  d is returned."""
    f = "nvfp4_gemm_sf"
    st = lib().nvfp4_gemm_sf(_ptr(a, _n(M, K) // 2, "a", f), _ptr(a_sf, _sf_bytes(M, K, sf_layout), "a_sf", f),
                             _ptr(b, _n(N, K) // 2, "b", f), _ptr(b_sf, _sf_bytes(N, K, sf_layout), "b_sf", f),
                             _ptr(alpha, 4, "alpha", f), _ptr(d, 2 * _n(M, N), "d", f), M, N, K, sf_layout,
                             _ptr(workspace, 0, "workspace", f), _bytes(workspace), _stream(stream))
    _check(st, f)
    return d


def nvfp4_grouped_gemm_sf(a, a_sf, b, b_sf, offsets, alpha, d, rows: int, N: int, K: int, E: int, sf_layout: int,
                          status=None, stream=None):
    """nvfp4_grouped_gemm with a_sf ([rows][K/16]) and b_sf ([E * N][K/16])
    in the scale layout sf_layout; see include/nvfp4.h.  d is returned."""
    f = "nvfp4_grouped_gemm_sf"
    st = lib().nvfp4_grouped_gemm_sf(_ptr(a, _n(rows, K) // 2, "a", f), _ptr(a_sf, _sf_bytes(rows, K, sf_layout), "a_sf", f),
                                     _ptr(b, _n(E, N, K) // 2, "b", f),
                                     _ptr(b_sf, _sf_bytes(_n(E, N), K, sf_layout), "b_sf", f),
                                     _ptr(offsets, 4 * _n(E + 1), "offsets", f), _ptr(alpha, 4 * _n(E), "alpha", f),
                                     _ptr(d, 2 * _n(rows, N), "d", f), rows, N, K, E, sf_layout,
                                     _ptr(status, 4, "status", f), _stream(stream))
    _check(st, f)
    return d


def nvfp4_grouped_gemm(a, a_sf, b, b_sf, offsets, alpha, d, rows: int, N: int, K: int, E: int,
                       workspace=None, status=None, stream=None):
    f = "nvfp4_grouped_gemm"
    st = lib().nvfp4_grouped_gemm(_ptr(a, _n(rows, K) // 2, "a", f), _ptr(a_sf, _n(rows, K) // 16, "a_sf", f),
                                  _ptr(b, _n(E, N, K) // 2, "b", f), _ptr(b_sf, _n(E, N, K) // 16, "b_sf", f),
                                  _ptr(offsets, 4 * _n(E + 1), "offsets", f), _ptr(alpha, 4 * _n(E), "alpha", f),
                                  _ptr(d, 2 * _n(rows, N), "d", f), rows, N, K, E,
                                  _ptr(workspace, 0, "workspace", f), _bytes(workspace),
                                  _ptr(status, 4, "status", f), _stream(stream))
    _check(st, "nvfp4_grouped_gemm")
    return d


def nvfp4_grouped_packed_size(N: int, K: int, E: int):
    """(code bytes, scale bytes) of the packed expert weights (0, 0 if unsupported)."""
    sf = ctypes.c_size_t(0)
    code = int(lib().nvfp4_grouped_packed_size(N, K, E, ctypes.byref(sf)))
    return code, int(sf.value)


def nvfp4_grouped_pack_b(b, b_sf, N: int, K: int, E: int, packed, packed_sf, stream=None):
    f = "nvfp4_grouped_pack_b"
    cb, sb = nvfp4_grouped_packed_size(N, K, E)
    st = lib().nvfp4_grouped_pack_b(_ptr(b, _n(E, N, K) // 2, "b", f), _ptr(b_sf, _n(E, N, K) // 16, "b_sf", f),
                                    N, K, E, _ptr(packed, cb, "packed", f), _ptr(packed_sf, sb, "packed_sf", f),
                                    _stream(stream))
    _check(st, "nvfp4_grouped_pack_b")
    return packed, packed_sf


def grouped_pack(b, b_sf, N: int, K: int, E: int, device="cuda"):
    """Allocate and fill the packed expert weights for nvfp4_grouped_gemm_packed."""
    import torch
    cb, sb = nvfp4_grouped_packed_size(N, K, E)
    if cb == 0:
        raise Nvfp4Error(4, "grouped_pack", f"N={N}, K={K}, E={E} cannot be packed (needs K % 512 == 0)")
    packed = torch.empty(cb, dtype=torch.uint8, device=device)
    packed_sf = torch.empty(sb, dtype=torch.uint8, device=device)
    return nvfp4_grouped_pack_b(b, b_sf, N, K, E, packed, packed_sf)


def nvfp4_grouped_gemm_packed(a, a_sf, packed, packed_sf, offsets, alpha, d, rows: int, N: int, K: int, E: int,
                              status=None, stream=None):
    f = "nvfp4_grouped_gemm_packed"
    cb, sb = nvfp4_grouped_packed_size(N, K, E)
    st = lib().nvfp4_grouped_gemm_packed(_ptr(a, _n(rows, K) // 2, "a", f), _ptr(a_sf, _n(rows, K) // 16, "a_sf", f),
                                         _ptr(packed, cb, "packed", f), _ptr(packed_sf, sb, "packed_sf", f),
                                         _ptr(offsets, 4 * _n(E + 1), "offsets", f),
                                         _ptr(alpha, 4 * _n(E), "alpha", f), _ptr(d, 2 * _n(rows, N), "d", f),
                                         rows, N, K, E, _ptr(status, 4, "status", f), _stream(stream))
    _check(st, "nvfp4_grouped_gemm_packed")
    return d


def nvfp4_grouped_gemm_fused(x, row_token, a_global_scale, b, b_sf, offsets, alpha, d, rows: int, T: int, N: int,
                             K: int, E: int, status=None, stream=None):
    """Grouped GEMM quantising bf16 activations x [T][K] on load: A row i is
    x[row_token[i]] (x[i] when row_token is None); b, b_sf as nvfp4_grouped_gemm."""
    f = "nvfp4_grouped_gemm_fused"
    st = lib().nvfp4_grouped_gemm_fused(_ptr(x, 2 * _n(T, K), "x", f), _ptr(row_token, 4 * _n(rows), "row_token", f),
                                        _ptr(a_global_scale, 4, "a_global_scale", f),
                                        _ptr(b, _n(E, N, K) // 2, "b", f), _ptr(b_sf, _n(E, N, K) // 16, "b_sf", f),
                                        _ptr(offsets, 4 * _n(E + 1), "offsets", f),
                                        _ptr(alpha, 4 * _n(E), "alpha", f), _ptr(d, 2 * _n(rows, N), "d", f),
                                        rows, T, N, K, E, _ptr(status, 4, "status", f), _stream(stream))
    _check(st, "nvfp4_grouped_gemm_fused")
    return d


def nvfp4_grouped_gemm_packed_fused(x, row_token, a_global_scale, packed, packed_sf, offsets, alpha, d, rows: int,
                                    T: int, N: int, K: int, E: int, status=None, stream=None):
    """nvfp4_grouped_gemm_fused on weights packed by nvfp4_grouped_pack_b."""
    f = "nvfp4_grouped_gemm_packed_fused"
    cb, sb = nvfp4_grouped_packed_size(N, K, E)
    st = lib().nvfp4_grouped_gemm_packed_fused(_ptr(x, 2 * _n(T, K), "x", f),
                                               _ptr(row_token, 4 * _n(rows), "row_token", f),
                                               _ptr(a_global_scale, 4, "a_global_scale", f),
                                               _ptr(packed, cb, "packed", f), _ptr(packed_sf, sb, "packed_sf", f),
                                               _ptr(offsets, 4 * _n(E + 1), "offsets", f),
                                               _ptr(alpha, 4 * _n(E), "alpha", f), _ptr(d, 2 * _n(rows, N), "d", f),
                                               rows, T, N, K, E, _ptr(status, 4, "status", f), _stream(stream))
    _check(st, "nvfp4_grouped_gemm_packed_fused")
    return d


def nvfp4_quantize_rows_bf16(x, row_token, gs, q, sf, rows: int, T: int, K: int, stream=None):
    """NVFP4 of bf16 rows x[row_token[i]] (x[i] when row_token is None)."""
    f = "nvfp4_quantize_rows_bf16"
    st = lib().nvfp4_quantize_rows_bf16(_ptr(x, 2 * _n(T, K), "x", f), _ptr(row_token, 4 * _n(rows), "row_token", f),
                                        _ptr(gs, 4, "gs", f), _ptr(q, _n(rows, K) // 2, "q", f),
                                        _ptr(sf, _n(rows, K) // 16, "sf", f), rows, T, K, _stream(stream))
    _check(st, "nvfp4_quantize_rows_bf16")
    return q, sf


def nvfp4_swiglu_quantize(gu, rows: int, I: int, gs, q, sf, stream=None):
    """h = silu(gate) * up of bf16 gu [rows][2I], quantised to NVFP4 (q, sf)."""
    f = "nvfp4_swiglu_quantize"
    st = lib().nvfp4_swiglu_quantize(_ptr(gu, 4 * _n(rows, I), "gu", f), rows, I, _ptr(gs, 4, "gs", f),
                                     _ptr(q, _n(rows, I) // 2, "q", f), _ptr(sf, _n(rows, I) // 16, "sf", f),
                                     _stream(stream))
    _check(st, "nvfp4_swiglu_quantize")
    return q, sf


def nvfp4_moe_combine(down, rows_of, weight, out, T: int, H: int, top_k: int, rows: int, stream=None):
    f = "nvfp4_moe_combine"
    st = lib().nvfp4_moe_combine(_ptr(down, 2 * _n(rows, H), "down", f), _ptr(rows_of, 4 * _n(T, top_k), "rows_of", f),
                                 _ptr(weight, 4 * _n(T, top_k), "weight", f), _ptr(out, 2 * _n(T, H), "out", f),
                                 T, H, top_k, rows, _stream(stream))
    _check(st, "nvfp4_moe_combine")
    return out


def nvfp4_moe_ffn_workspace_size(T: int, H: int, I: int, top_k: int) -> int:
    return int(lib().nvfp4_moe_ffn_workspace_size(T, H, I, top_k))


def nvfp4_moe_ffn(x, gs_x, row_token, offsets, w_gu, w_gu_sf, alpha_gu, gs_h, w_d, w_d_sf, alpha_d, token_rows,
                  token_weight, out, T: int, H: int, I: int, E: int, top_k: int, workspace, status=None,
                  stream=None):
    """One MoE layer's experts: fused gate/up grouped GEMM, SwiGLU + NVFP4,
    down grouped GEMM, weighted combine (weights packed by nvfp4_grouped_pack_b)."""
    f = "nvfp4_moe_ffn"
    gcb, gsb = nvfp4_grouped_packed_size(2 * I, H, E)
    dcb, dsb = nvfp4_grouped_packed_size(H, I, E)
    rows = _n(T, top_k)
    st = lib().nvfp4_moe_ffn(_ptr(x, 2 * _n(T, H), "x", f), _ptr(gs_x, 4, "gs_x", f),
                             _ptr(row_token, 4 * rows, "row_token", f), _ptr(offsets, 4 * _n(E + 1), "offsets", f),
                             _ptr(w_gu, gcb, "w_gu", f), _ptr(w_gu_sf, gsb, "w_gu_sf", f),
                             _ptr(alpha_gu, 4 * _n(E), "alpha_gu", f), _ptr(gs_h, 4, "gs_h", f),
                             _ptr(w_d, dcb, "w_d", f), _ptr(w_d_sf, dsb, "w_d_sf", f),
                             _ptr(alpha_d, 4 * _n(E), "alpha_d", f), _ptr(token_rows, 4 * rows, "token_rows", f),
                             _ptr(token_weight, 4 * rows, "token_weight", f), _ptr(out, 2 * _n(T, H), "out", f),
                             T, H, I, E, top_k, _ptr(workspace, 0, "workspace", f), _bytes(workspace),
                             _ptr(status, 4, "status", f), _stream(stream))
    _check(st, "nvfp4_moe_ffn")
    return out


def nvfp4_scales_128x4_size(rows: int, K: int) -> int:
    return int(lib().nvfp4_scales_128x4_size(rows, K))


def nvfp4_scales_to_128x4(sf, tiled, rows: int, K: int, stream=None):
    """Linear [rows][K/16] scales -> the 128 x 4 tiled layout."""
    f = "nvfp4_scales_to_128x4"
    _check(lib().nvfp4_scales_to_128x4(_ptr(sf, _n(rows, K) // 16, "sf", f),
                                       _ptr(tiled, nvfp4_scales_128x4_size(rows, K), "tiled", f), rows, K,
                                       _stream(stream)), f)
    return tiled


def nvfp4_scales_from_128x4(tiled, sf, rows: int, K: int, stream=None):
    """The 128 x 4 tiled layout -> linear [rows][K/16] scales."""
    f = "nvfp4_scales_from_128x4"
    _check(lib().nvfp4_scales_from_128x4(_ptr(tiled, nvfp4_scales_128x4_size(rows, K), "tiled", f),
                                         _ptr(sf, _n(rows, K) // 16, "sf", f), rows, K, _stream(stream)), f)
    return sf


def nvfp4_scales_8x4_size(rows: int, K: int) -> int:
    return int(lib().nvfp4_scales_8x4_size(rows, K))


def nvfp4_scales_to_8x4(sf, tiled, rows: int, K: int, stream=None):
    """Linear [rows][K/16] scales -> the 8 x 4 tiled layout."""
    f = "nvfp4_scales_to_8x4"
    _check(lib().nvfp4_scales_to_8x4(_ptr(sf, _n(rows, K) // 16, "sf", f),
                                     _ptr(tiled, nvfp4_scales_8x4_size(rows, K), "tiled", f), rows, K,
                                     _stream(stream)), f)
    return tiled


def nvfp4_scales_from_8x4(tiled, sf, rows: int, K: int, stream=None):
    """The 8 x 4 tiled layout -> linear [rows][K/16] scales."""
    f = "nvfp4_scales_from_8x4"
    _check(lib().nvfp4_scales_from_8x4(_ptr(tiled, nvfp4_scales_8x4_size(rows, K), "tiled", f),
                                       _ptr(sf, _n(rows, K) // 16, "sf", f), rows, K, _stream(stream)), f)
    return sf


def nvfp4_quantize(x, R: int, K: int, global_scale, q, sf, stream=None):
    f = "nvfp4_quantize"
    st = lib().nvfp4_quantize(_ptr(x, 4 * _n(R, K), "x", f), R, K, _ptr(global_scale, 4, "global_scale", f),
                              _ptr(q, _n(R, K) // 2, "q", f), _ptr(sf, _n(R, K) // 16, "sf", f), _stream(stream))
    _check(st, "nvfp4_quantize")
    return q, sf


def nvfp4_global_scale(x, n: int, gs, stream=None):
    f = "nvfp4_global_scale"
    st = lib().nvfp4_global_scale(_ptr(x, 4 * _n(n), "x", f), n, _ptr(gs, 4, "gs", f), _stream(stream))
    _check(st, "nvfp4_global_scale")
    return gs


def nvfp4_alpha_from_scales(gs_a, gs_b, alpha, count: int, stream=None):
    f = "nvfp4_alpha_from_scales"
    st = lib().nvfp4_alpha_from_scales(_ptr(gs_a, 4, "gs_a", f), _ptr(gs_b, 4 * _n(count), "gs_b", f),
                                       _ptr(alpha, 4 * _n(count), "alpha", f), count, _stream(stream))
    _check(st, "nvfp4_alpha_from_scales")
    return alpha
