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
    "nvfp4_gemm_workspace_size": (_sz, [_i64, _i64, _i64]),
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
    "nvfp4_quantize": (ctypes.c_int, [_vp, _i64, _i64, _vp, _vp, _vp, _vp]),
    "nvfp4_global_scale": (ctypes.c_int, [_vp, _i64, _vp, _vp]),
    "nvfp4_alpha_from_scales": (ctypes.c_int, [_vp, _vp, _vp, _i32, _vp]),
    "nvfp4_gemm_plan": (ctypes.c_char_p, [_i64, _i64, _i64]),
    "nvfp4_mx_gemm": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _sz, _vp]),
    "nvfp4_mx_gemm_workspace_size": (_sz, [_i64, _i64, _i64]),
    "nvfp4_mx_gemm_plan": (ctypes.c_char_p, [_i64, _i64, _i64]),
    "nvfp4_last_error": (ctypes.c_char_p, []),
}

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


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is not None:
        return ctypes.c_void_p(stream)
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(status: int, fn: str):
    if status != 0:
        raise Nvfp4Error(status, fn, lib().nvfp4_last_error().decode())


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
    st = lib().nvfp4_workspace_init(_ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
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
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().nvfp4_mx_gemm(_ptr(a), _ptr(a_sf), _ptr(b), _ptr(b_sf), _ptr(alpha), _ptr(d), M, N, K,
                             _ptr(workspace), ws_bytes, _stream(stream))
    _check(st, "nvfp4_mx_gemm")
    return d


def nvfp4_grouped_workspace_size(rows: int, N: int, K: int, E: int) -> int:
    return int(lib().nvfp4_grouped_workspace_size(rows, N, K, E))


def nvfp4_gemm(a, a_sf, b, b_sf, alpha, d, M: int, N: int, K: int, workspace=None, stream=None):
    """D = bf16(alpha * dequant(A) @ dequant(B)^T); see include/nvfp4.h.
    a: uint8 [M][K/2], a_sf: uint8 [M][K/16], b: uint8 [N][K/2],
    b_sf: uint8 [N][K/16], alpha: fp32 device scalar tensor or None,
    d: caller-allocated [M][N] bf16 (or int16/uint16) tensor, returned."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().nvfp4_gemm(_ptr(a), _ptr(a_sf), _ptr(b), _ptr(b_sf), _ptr(alpha), _ptr(d), M, N, K,
                          _ptr(workspace), ws_bytes, _stream(stream))
    _check(st, "nvfp4_gemm")
    return d


def nvfp4_grouped_gemm(a, a_sf, b, b_sf, offsets, alpha, d, rows: int, N: int, K: int, E: int,
                       workspace=None, status=None, stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().nvfp4_grouped_gemm(_ptr(a), _ptr(a_sf), _ptr(b), _ptr(b_sf), _ptr(offsets), _ptr(alpha), _ptr(d),
                                  rows, N, K, E, _ptr(workspace), ws_bytes, _ptr(status), _stream(stream))
    _check(st, "nvfp4_grouped_gemm")
    return d


def nvfp4_grouped_packed_size(N: int, K: int, E: int):
    """(code bytes, scale bytes) of the packed expert weights (0, 0 if unsupported)."""
    sf = ctypes.c_size_t(0)
    code = int(lib().nvfp4_grouped_packed_size(N, K, E, ctypes.byref(sf)))
    return code, int(sf.value)


def nvfp4_grouped_pack_b(b, b_sf, N: int, K: int, E: int, packed, packed_sf, stream=None):
    st = lib().nvfp4_grouped_pack_b(_ptr(b), _ptr(b_sf), N, K, E, _ptr(packed), _ptr(packed_sf), _stream(stream))
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
    st = lib().nvfp4_grouped_gemm_packed(_ptr(a), _ptr(a_sf), _ptr(packed), _ptr(packed_sf), _ptr(offsets),
                                         _ptr(alpha), _ptr(d), rows, N, K, E, _ptr(status), _stream(stream))
    _check(st, "nvfp4_grouped_gemm_packed")
    return d


def nvfp4_grouped_gemm_fused(x, row_token, a_global_scale, b, b_sf, offsets, alpha, d, rows: int, T: int, N: int,
                             K: int, E: int, status=None, stream=None):
    """Grouped GEMM quantising bf16 activations x [T][K] on load: A row i is
    x[row_token[i]] (x[i] when row_token is None); b, b_sf as nvfp4_grouped_gemm."""
    st = lib().nvfp4_grouped_gemm_fused(_ptr(x), _ptr(row_token), _ptr(a_global_scale), _ptr(b), _ptr(b_sf),
                                        _ptr(offsets), _ptr(alpha), _ptr(d), rows, T, N, K, E, _ptr(status),
                                        _stream(stream))
    _check(st, "nvfp4_grouped_gemm_fused")
    return d


def nvfp4_grouped_gemm_packed_fused(x, row_token, a_global_scale, packed, packed_sf, offsets, alpha, d, rows: int,
                                    T: int, N: int, K: int, E: int, status=None, stream=None):
    """nvfp4_grouped_gemm_fused on weights packed by nvfp4_grouped_pack_b."""
    st = lib().nvfp4_grouped_gemm_packed_fused(_ptr(x), _ptr(row_token), _ptr(a_global_scale), _ptr(packed),
                                               _ptr(packed_sf), _ptr(offsets), _ptr(alpha), _ptr(d), rows, T, N, K,
                                               E, _ptr(status), _stream(stream))
    _check(st, "nvfp4_grouped_gemm_packed_fused")
    return d


def nvfp4_quantize_rows_bf16(x, row_token, gs, q, sf, rows: int, T: int, K: int, stream=None):
    """NVFP4 of bf16 rows x[row_token[i]] (x[i] when row_token is None)."""
    st = lib().nvfp4_quantize_rows_bf16(_ptr(x), _ptr(row_token), _ptr(gs), _ptr(q), _ptr(sf), rows, T, K,
                                        _stream(stream))
    _check(st, "nvfp4_quantize_rows_bf16")
    return q, sf


def nvfp4_swiglu_quantize(gu, rows: int, I: int, gs, q, sf, stream=None):
    """h = silu(gate) * up of bf16 gu [rows][2I], quantised to NVFP4 (q, sf)."""
    st = lib().nvfp4_swiglu_quantize(_ptr(gu), rows, I, _ptr(gs), _ptr(q), _ptr(sf), _stream(stream))
    _check(st, "nvfp4_swiglu_quantize")
    return q, sf


def nvfp4_moe_combine(down, rows_of, weight, out, T: int, H: int, top_k: int, rows: int, stream=None):
    st = lib().nvfp4_moe_combine(_ptr(down), _ptr(rows_of), _ptr(weight), _ptr(out), T, H, top_k, rows,
                                 _stream(stream))
    _check(st, "nvfp4_moe_combine")
    return out


def nvfp4_moe_ffn_workspace_size(T: int, H: int, I: int, top_k: int) -> int:
    return int(lib().nvfp4_moe_ffn_workspace_size(T, H, I, top_k))


def nvfp4_moe_ffn(x, gs_x, row_token, offsets, w_gu, w_gu_sf, alpha_gu, gs_h, w_d, w_d_sf, alpha_d, token_rows,
                  token_weight, out, T: int, H: int, I: int, E: int, top_k: int, workspace, status=None,
                  stream=None):
    """One MoE layer's experts: fused gate/up grouped GEMM, SwiGLU + NVFP4,
    down grouped GEMM, weighted combine (weights packed by nvfp4_grouped_pack_b)."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().nvfp4_moe_ffn(_ptr(x), _ptr(gs_x), _ptr(row_token), _ptr(offsets), _ptr(w_gu), _ptr(w_gu_sf),
                             _ptr(alpha_gu), _ptr(gs_h), _ptr(w_d), _ptr(w_d_sf), _ptr(alpha_d), _ptr(token_rows),
                             _ptr(token_weight), _ptr(out), T, H, I, E, top_k, _ptr(workspace), ws_bytes,
                             _ptr(status), _stream(stream))
    _check(st, "nvfp4_moe_ffn")
    return out


def nvfp4_scales_128x4_size(rows: int, K: int) -> int:
    return int(lib().nvfp4_scales_128x4_size(rows, K))


def nvfp4_scales_to_128x4(sf, tiled, rows: int, K: int, stream=None):
    """Linear [rows][K/16] scales -> the 128 x 4 tiled layout."""
    _check(lib().nvfp4_scales_to_128x4(_ptr(sf), _ptr(tiled), rows, K, _stream(stream)), "nvfp4_scales_to_128x4")
    return tiled


def nvfp4_scales_from_128x4(tiled, sf, rows: int, K: int, stream=None):
    """The 128 x 4 tiled layout -> linear [rows][K/16] scales."""
    _check(lib().nvfp4_scales_from_128x4(_ptr(tiled), _ptr(sf), rows, K, _stream(stream)),
           "nvfp4_scales_from_128x4")
    return sf


def nvfp4_quantize(x, R: int, K: int, global_scale, q, sf, stream=None):
    st = lib().nvfp4_quantize(_ptr(x), R, K, _ptr(global_scale), _ptr(q), _ptr(sf), _stream(stream))
    _check(st, "nvfp4_quantize")
    return q, sf


def nvfp4_global_scale(x, n: int, gs, stream=None):
    st = lib().nvfp4_global_scale(_ptr(x), n, _ptr(gs), _stream(stream))
    _check(st, "nvfp4_global_scale")
    return gs


def nvfp4_alpha_from_scales(gs_a, gs_b, alpha, count: int, stream=None):
    st = lib().nvfp4_alpha_from_scales(_ptr(gs_a), _ptr(gs_b), _ptr(alpha), count, _stream(stream))
    _check(st, "nvfp4_alpha_from_scales")
    return alpha
