"""Python binding of libmxg, the MI355X block-scaled grouped-GEMM / MoE library.

Argument marshalling only: every function forwards torch tensors' device pointers to
the C ABI of ``include/mxg.h`` (same names) on torch's current HIP stream and raises
``MxgError`` on a non-zero status.  torch provides device memory and streams; all
computation happens in the library's HIP kernels.  There is no fallback: if
``libmxg.so`` is missing, importing the binding's entry points raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmxg.so")

MXG_OK, MXG_ERR_INVALID_ARG, MXG_ERR_UNSUPPORTED, MXG_ERR_WORKSPACE, MXG_ERR_HIP = range(5)
MXG_E2M1, MXG_E4M3, MXG_BF16, MXG_F32, MXG_E4M3_POW2 = 1, 2, 3, 4, 5
MXG_MOE_FP8_BLOCK128, MXG_MOE_NVFP4, MXG_MOE_FP8_BLOCK128_F32H = 1, 2, 3
MXG_W13_STACKED, MXG_W13_INTERLEAVED16 = 0, 16
MXG_MAX_GROUPS = 32


class MxgError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (status {status})")
        self.status = status


class GroupDesc(ctypes.Structure):
    _fields_ = [("M", ctypes.c_int), ("N", ctypes.c_int), ("K", ctypes.c_int), ("ldc", ctypes.c_int),
                ("alpha", ctypes.c_float), ("a", ctypes.c_void_p), ("a_sf", ctypes.c_void_p),
                ("b", ctypes.c_void_p), ("b_sf", ctypes.c_void_p), ("out", ctypes.c_void_p)]


class MoeDesc(ctypes.Structure):
    _fields_ = [("precision", ctypes.c_int), ("T", ctypes.c_int), ("H", ctypes.c_int), ("I", ctypes.c_int),
                ("E", ctypes.c_int), ("top_k", ctypes.c_int), ("max_m", ctypes.c_int),
                ("x", ctypes.c_void_p), ("x_scale", ctypes.c_void_p), ("g_x", ctypes.c_float),
                ("w13", ctypes.c_void_p), ("w13_scale", ctypes.c_void_p), ("g_w13", ctypes.c_void_p),
                ("w2", ctypes.c_void_p), ("w2_scale", ctypes.c_void_p), ("g_w2", ctypes.c_void_p),
                ("g_h", ctypes.c_float),
                ("topk_ids", ctypes.c_void_p), ("topk_w", ctypes.c_void_p), ("masked_m", ctypes.c_void_p),
                ("row", ctypes.c_void_p), ("y", ctypes.c_void_p), ("dbg_h", ctypes.c_void_p),
                ("w13_layout", ctypes.c_int), ("dbg_g1", ctypes.c_void_p)]


_LIB = None
_P, _I, _L, _F, _SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_long, ctypes.c_float, ctypes.c_size_t

SIGNATURES = {
    "mxg_status_string": (ctypes.c_char_p, [_I]),
    "mxg_last_error": (ctypes.c_char_p, []),
    "mxg_version": (_I, []),
    "mx_grouped_gemm_masked": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I, _P]),
    "mx_grouped_gemm": (_I, [_P, _I, _I, _I, _I, _I, _I, _P]),
    "mx_grouped_gemm_contiguous": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I, _P]),
    "moe_dispatch_contiguous": (_I, [_P, _I, _I, _I, _I, _P, _P, _P, _P]),
    "mx_gemv_nvfp4_w4a16": (_I, [_P, _I, _I, _P, _P, _F, _P, _I, _I, _I, _P]),
    "mx_quantize_nvfp4": (_I, [_P, _I, _L, _I, _F, _P, _P, _P]),
    "moe_route_noaux": (_I, [_P, _P, _I, _I, _I, _I, _I, _F, _P, _P, _P]),
    "moe_dispatch": (_I, [_P, _I, _I, _I, _I, _P, _P, _P, _P]),
    "moe_quantize_gather_nvfp4": (_I, [_P, _I, _I, _F, _P, _P, _I, _I, _I, _P, _P, _P]),
    "moe_dispatch_quantize_gather_nvfp4": (_I, [_P, _I, _I, _F, _P, _I, _I, _I, _P, _P, _P, _P, _P]),
    "moe_interleave_w13": (_I, [_P, _P, _I, _I, _I, _P]),
    "moe_expert_forward_workspace_size": (_SZ, [_P]),
    "moe_expert_forward_workspace_layout": (_I, [_P, _P]),
    "moe_expert_forward": (_I, [_P, _P, _SZ, _P]),
    "moe_expert_forward_noalloc": (_I, [_P, _P]),
}


def lib():
    """Load libmxg.so (torch first, so the library binds to torch's HIP runtime)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = handle
    return _LIB


def _check(status: int):
    if status != MXG_OK:
        raise MxgError(status, lib().mxg_last_error().decode())


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def mx_grouped_gemm_masked(a, a_sf, b, b_sf, alpha, masked_m, out, cu_limit=0, stream=None,
                           ab_dtype=MXG_E2M1, sf_dtype=MXG_E4M3, sf_vec_size=16):
    """Masked grouped NVFP4 NT GEMM.  a [G, max_m, K/2] u8, a_sf [G, max_m, K/16] u8,
    b [G, N, K/2], b_sf [G, N, K/16], alpha [G] f32 or None, masked_m [G] i32,
    out [G, max_m, N] bf16 or f32."""
    G, max_m, half_k = a.shape
    N = b.shape[1]
    c_dtype = {torch.bfloat16: MXG_BF16, torch.float32: MXG_F32}.get(out.dtype, 0)
    _check(lib().mx_grouped_gemm_masked(_ptr(a), _ptr(a_sf), _ptr(b), _ptr(b_sf), _ptr(alpha),
                                        _ptr(masked_m), _ptr(out), G, max_m, N, 2 * half_k, ab_dtype,
                                        sf_dtype, c_dtype, sf_vec_size, cu_limit, _stream(stream)))
    return out


def mx_grouped_gemm_contiguous(a, a_sf, b, b_sf, alpha, group_start, count, out, cu_limit=0, stream=None):
    """Contiguous-layout grouped NVFP4 NT GEMM.  a [M_total, K/2] u8, a_sf [M_total, K/16] u8,
    b [G, N, K/2], b_sf [G, N, K/16], alpha [G] f32 or None, group_start [G + 1] i32,
    count [G] i32, out [M_total, N] bf16 or f32."""
    M_total, half_k = a.shape
    G, N = b.shape[0], b.shape[1]
    c_dtype = {torch.bfloat16: MXG_BF16, torch.float32: MXG_F32}.get(out.dtype, 0)
    _check(lib().mx_grouped_gemm_contiguous(_ptr(a), _ptr(a_sf), _ptr(b), _ptr(b_sf), _ptr(alpha),
                                            _ptr(group_start), _ptr(count), _ptr(out), G, M_total, N,
                                            2 * half_k, MXG_E2M1, MXG_E4M3, c_dtype, 16, cu_limit,
                                            _stream(stream)))
    return out


def mx_grouped_gemm(groups, out_dtype=torch.bfloat16, cu_limit=0, stream=None, sf_dtype=MXG_E4M3):
    """Heterogeneous grouped NVFP4 NT GEMM.  groups: list of dicts with M, N, K, alpha,
    a, a_sf, b, b_sf, out (tensors) and optional ldc.  sf_dtype=MXG_E4M3_POW2 declares
    every scale byte a positive power of two (the fp4-MFMA path)."""
    G = len(groups)
    arr = (GroupDesc * max(G, 1))()
    for i, g in enumerate(groups):
        arr[i] = GroupDesc(g["M"], g["N"], g["K"], g.get("ldc", 0), float(g["alpha"]),
                           _ptr(g["a"]), _ptr(g["a_sf"]), _ptr(g["b"]), _ptr(g["b_sf"]), _ptr(g["out"]))
    c_dtype = {torch.bfloat16: MXG_BF16, torch.float32: MXG_F32}.get(out_dtype, 0)
    _check(lib().mx_grouped_gemm(arr, G, MXG_E2M1, sf_dtype, c_dtype, 16, cu_limit, _stream(stream)))


def mx_gemv_nvfp4_w4a16(x, w, w_sf, g_w, out=None, out_dtype=torch.bfloat16, cu_limit=0, stream=None):
    """NVFP4-weight x bf16-activation GEMV: x [M, K] bf16, w [N, K/2] u8, w_sf [N, K/16] u8,
    g_w the weights' global scale; returns out [M, N] (bf16 or f32)."""
    M, K = x.shape
    N = w.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=x.device)
    c_dtype = {torch.bfloat16: MXG_BF16, torch.float32: MXG_F32}.get(out.dtype, 0)
    _check(lib().mx_gemv_nvfp4_w4a16(_ptr(x), M, K, _ptr(w), _ptr(w_sf), float(g_w), _ptr(out), N, c_dtype,
                                     cu_limit, _stream(stream)))
    return out


def mx_quantize_nvfp4(x, g, codes=None, sf=None, stream=None):
    """NVFP4-quantize rows of x [..., K] (bf16 or f32) with global scale g."""
    K = x.shape[-1]
    rows = x.numel() // K
    if codes is None:
        codes = torch.empty(x.shape[:-1] + (K // 2,), dtype=torch.uint8, device=x.device)
    if sf is None:
        sf = torch.empty(x.shape[:-1] + (K // 16,), dtype=torch.uint8, device=x.device)
    x_dtype = {torch.bfloat16: MXG_BF16, torch.float32: MXG_F32}.get(x.dtype, 0)
    _check(lib().mx_quantize_nvfp4(_ptr(x), x_dtype, rows, K, float(g), _ptr(codes), _ptr(sf),
                                   _stream(stream)))
    return codes, sf


def moe_route_noaux(logits, bias, n_group, topk_group, top_k, rsf, ids=None, w=None, stream=None):
    T, E = logits.shape
    if ids is None:
        ids = torch.empty((T, top_k), dtype=torch.int32, device=logits.device)
    if w is None:
        w = torch.empty((T, top_k), dtype=torch.float32, device=logits.device)
    _check(lib().moe_route_noaux(_ptr(logits), _ptr(bias), T, E, n_group, topk_group, top_k, float(rsf),
                                 _ptr(ids), _ptr(w), _stream(stream)))
    return ids, w


def moe_dispatch(ids, E, max_m, masked_m=None, row=None, stream=None, offsets=None, with_offsets=False):
    """Masked-layout dispatch: returns (masked_m, row), or (masked_m, row, offsets) when
    with_offsets or an offsets tensor [E + 1] is given."""
    T, k = ids.shape
    if masked_m is None:
        masked_m = torch.empty((E,), dtype=torch.int32, device=ids.device)
    if row is None:
        row = torch.empty((T, k), dtype=torch.int32, device=ids.device)
    if offsets is None and with_offsets:
        offsets = torch.empty((E + 1,), dtype=torch.int32, device=ids.device)
    _check(lib().moe_dispatch(_ptr(ids), T, E, k, max_m, _ptr(masked_m), _ptr(row), _ptr(offsets),
                              _stream(stream)))
    return (masked_m, row) if offsets is None else (masked_m, row, offsets)


def moe_dispatch_contiguous(ids, E, align, group_start=None, count=None, row=None, stream=None):
    T, k = ids.shape
    if group_start is None:
        group_start = torch.empty((E + 1,), dtype=torch.int32, device=ids.device)
    if count is None:
        count = torch.empty((E,), dtype=torch.int32, device=ids.device)
    if row is None:
        row = torch.empty((T, k), dtype=torch.int32, device=ids.device)
    _check(lib().moe_dispatch_contiguous(_ptr(ids), T, E, k, align, _ptr(group_start), _ptr(count), _ptr(row),
                                         _stream(stream)))
    return group_start, count, row


def moe_quantize_gather_nvfp4(x, g_x, ids, row, E, max_m, a=None, a_sf=None, stream=None):
    T, H = x.shape
    k = ids.shape[1]
    if a is None:
        a = torch.empty((E, max_m, H // 2), dtype=torch.uint8, device=x.device)
    if a_sf is None:
        a_sf = torch.empty((E, max_m, H // 16), dtype=torch.uint8, device=x.device)
    _check(lib().moe_quantize_gather_nvfp4(_ptr(x.view(torch.uint16) if x.dtype == torch.bfloat16 else x),
                                           T, H, float(g_x), _ptr(ids), _ptr(row), k, E, max_m,
                                           _ptr(a), _ptr(a_sf), _stream(stream)))
    return a, a_sf


def moe_dispatch_quantize_gather_nvfp4(x, g_x, ids, E, max_m, masked_m=None, row=None, a=None, a_sf=None,
                                       stream=None):
    """moe_dispatch followed by moe_quantize_gather_nvfp4 (one launch for small batches)."""
    T, H = x.shape
    k = ids.shape[1]
    if masked_m is None:
        masked_m = torch.empty((E,), dtype=torch.int32, device=x.device)
    if row is None:
        row = torch.empty((T, k), dtype=torch.int32, device=x.device)
    if a is None:
        a = torch.empty((E, max_m, H // 2), dtype=torch.uint8, device=x.device)
    if a_sf is None:
        a_sf = torch.empty((E, max_m, H // 16), dtype=torch.uint8, device=x.device)
    _check(lib().moe_dispatch_quantize_gather_nvfp4(_ptr(x.view(torch.uint16) if x.dtype == torch.bfloat16 else x),
                                                    T, H, float(g_x), _ptr(ids), k, E, max_m, _ptr(masked_m),
                                                    _ptr(row), _ptr(a), _ptr(a_sf), _stream(stream)))
    return masked_m, row, a, a_sf


def make_moe_desc(precision, T, H, I, E, top_k, max_m, x, w13, w13_scale, w2, w2_scale,
                  topk_ids, topk_w, masked_m, row, y, x_scale=None, g_x=0.0, g_w13=None, g_w2=None,
                  g_h=0.0, dbg_h=None, w13_layout=0, dbg_g1=None):
    return MoeDesc(precision, T, H, I, E, top_k, max_m, _ptr(x), _ptr(x_scale), float(g_x),
                   _ptr(w13), _ptr(w13_scale), _ptr(g_w13), _ptr(w2), _ptr(w2_scale), _ptr(g_w2),
                   float(g_h), _ptr(topk_ids), _ptr(topk_w), _ptr(masked_m), _ptr(row), _ptr(y),
                   _ptr(dbg_h), int(w13_layout), _ptr(dbg_g1))


def moe_interleave_w13(src, dst=None, stream=None):
    """Stacked W13 rows (codes [E, 2I, H/2] or scales [E, 2I, H/16], uint8) into the
    16-row gate/up-interleaved order (MXG_W13_INTERLEAVED16)."""
    E, two_i, row_bytes = src.shape
    if dst is None:
        dst = torch.empty_like(src)
    _check(lib().moe_interleave_w13(_ptr(src), _ptr(dst), E, two_i // 2, row_bytes, _stream(stream)))
    return dst


def moe_expert_forward_workspace_size(desc: MoeDesc) -> int:
    n = lib().moe_expert_forward_workspace_size(ctypes.byref(desc))
    if n == 0:
        _check(MXG_ERR_INVALID_ARG)
    return n


def moe_expert_forward_workspace_layout(desc: MoeDesc):
    off = (ctypes.c_size_t * 6)()
    _check(lib().moe_expert_forward_workspace_layout(ctypes.byref(desc), off))
    return list(off)


def moe_expert_forward(desc: MoeDesc, ws, stream=None):
    _check(lib().moe_expert_forward(ctypes.byref(desc), _ptr(ws), ws.numel() * ws.element_size(),
                                    _stream(stream)))


def moe_expert_forward_noalloc(desc: MoeDesc, stream=None):
    """moe_expert_forward on the library's own device scratch (no workspace argument)."""
    _check(lib().moe_expert_forward_noalloc(ctypes.byref(desc), _stream(stream)))
