"""Plain CPU oracle for the NVFP4 / FP8 block-scaled grouped GEMM and the MoE expert path.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no code with
the GPU library; the arithmetic lives in ``oracle.c`` (fp64 sums, exact decode tables
built from bit fields, nearest-search encoders, a scalar router).  This module only
marshals numpy arrays into it and adds the few fp64 elementwise steps (combine) that
are clearer in numpy.

Every function is pinned by ``tests/test_oracle_*.py`` against brute force, closed
forms, invariants or library routines.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_SO = os.path.join(_HERE, "liboracle.so")
_LIB = None

CFLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-fPIC", "-shared"]


def build() -> str:
    """Compile oracle.c with gcc (no fast-math, no FMA contraction) into liboracle.so."""
    tmp = _SO + ".tmp"
    subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
    os.replace(tmp, _SO)
    return _SO


_P = ctypes.c_void_p
_I = ctypes.c_int
_L = ctypes.c_long
_D = ctypes.c_double
_F = ctypes.c_float


def _lib():
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(_SO):
        build()
    lib = ctypes.CDLL(_SO)
    sig = {
        "orc_init": (None, []),
        "orc_e2m1_value": (_D, [_I]),
        "orc_e4m3_value": (_D, [_I]),
        "orc_encode_e2m1": (_I, [_D]),
        "orc_encode_e4m3_sat": (_I, [_D]),
        "orc_bf16_bits": (ctypes.c_uint16, [_D]),
        "orc_bf16_value": (_D, [ctypes.c_uint16]),
        "orc_bf16_bits_array": (None, [_P, _L, _P]),
        "orc_encode_e2m1_array": (None, [_P, _L, _P]),
        "orc_encode_e4m3_array": (None, [_P, _L, _P]),
        "orc_nvfp4_row_dot": (None, [_P, _P, _L, _P, _P, _I, _I, _D, _P, _P]),
        "orc_gemm_nvfp4_rows": (None, [_P, _P, _P, _I, _P, _P, _I, _I, _D, _P, _P]),
        "orc_gemm_nvfp4_masked": (None, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _P, _P, _P]),
        "orc_gemm_fp8_block": (None, [_P, _P, _P, _I, _P, _P, _I, _I, _P, _P]),
        "orc_gemm_dense_fp8w": (None, [_P, _I, _P, _P, _I, _I, _P, _P]),
        "orc_gemv_nvfp4_w4a16": (None, [_P, _I, _P, _P, _I, _I, _D, _P, _P]),
        "orc_quantize_nvfp4": (None, [_P, _L, _I, _F, _P, _P]),
        "orc_route_noaux": (None, [_P, _P, _I, _I, _I, _I, _I, _F, _P, _P]),
        "orc_dispatch": (None, [_P, _I, _I, _I, _I, _P, _P]),
        "orc_swiglu": (None, [_P, _I, _I, _P]),
        "orc_num_threads": (_I, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    lib.orc_init()
    _LIB = lib
    return lib


def _c(a, dtype):
    """C-contiguous array of the given dtype (no copy when already so)."""
    return np.ascontiguousarray(a, dtype=dtype)


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


# ----------------------------------------------------------------------------- formats
def e2m1_value(code: int) -> float:
    return _lib().orc_e2m1_value(int(code))


def e4m3_value(code: int) -> float:
    return _lib().orc_e4m3_value(int(code))


def e2m1_table() -> np.ndarray:
    return np.array([e2m1_value(c) for c in range(16)])


def e4m3_table() -> np.ndarray:
    return np.array([e4m3_value(c) for c in range(256)])


def encode_e2m1(v) -> np.ndarray:
    v = _c(v, np.float64)
    out = np.empty(v.shape, np.uint8)
    _lib().orc_encode_e2m1_array(_p(v), v.size, _p(out))
    return out


def encode_e4m3_sat(v) -> np.ndarray:
    v = _c(v, np.float64)
    out = np.empty(v.shape, np.uint8)
    _lib().orc_encode_e4m3_array(_p(v), v.size, _p(out))
    return out


def bf16_bits(v) -> np.ndarray:
    """bf16 bit patterns (uint16) of fp64 values, rounded once to nearest even."""
    v = _c(v, np.float64)
    out = np.empty(v.shape, np.uint16)
    _lib().orc_bf16_bits_array(_p(v), v.size, _p(out))
    return out


def bf16_value(bits) -> np.ndarray:
    bits = _c(bits, np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def nvfp4_decode(codes, sf) -> np.ndarray:
    """Decoded values dec[r, k] = e2m1(code) * e4m3(scale of k's 16-block), fp64."""
    codes = _c(codes, np.uint8)
    sf = _c(sf, np.uint8)
    lo = codes & 15
    hi = codes >> 4
    nib = np.stack([lo, hi], axis=-1).reshape(*codes.shape[:-1], codes.shape[-1] * 2)
    vals = e2m1_table()[nib]
    scales = np.repeat(e4m3_table()[sf], 16, axis=-1)
    return vals * scales


# ----------------------------------------------------------------------------- GEMMs
def gemm_nvfp4_masked(a, a_sf, b, b_sf, alpha, masked_m, max_m, N, K, out=None):
    """Masked grouped NVFP4 NT GEMM.  Returns (y, s, out): y/s fp64 [G,max_m,N] (NaN in
    rows not computed), out uint16 bf16 bits; ``out`` (if given) keeps its content in
    rows at or beyond masked_m."""
    lib = _lib()
    G = len(masked_m)
    a = _c(a, np.uint8); a_sf = _c(a_sf, np.uint8); b = _c(b, np.uint8); b_sf = _c(b_sf, np.uint8)
    alpha = None if alpha is None else _c(alpha, np.float32)
    mm = _c(masked_m, np.int32)
    y = np.full((G, max_m, N), np.nan)
    s = np.full((G, max_m, N), np.nan)
    if out is None:
        out = np.zeros((G, max_m, N), np.uint16)
    else:
        out = _c(out, np.uint16).copy()
    lib.orc_gemm_nvfp4_masked(_p(a), _p(a_sf), _p(b), _p(b_sf), _p(alpha), _p(mm), G, max_m, N, K,
                              _p(y), _p(s), _p(out))
    return y, s, out


def nvfp4_row_dot(a, a_sf, a_row, b, b_sf, K, alpha=1.0):
    """One NVFP4 A row (row index a_row of [rows, K] codes/scales) against every row of B.
    Returns (y, s) fp64 [nb]."""
    lib = _lib()
    a = _c(a, np.uint8); a_sf = _c(a_sf, np.uint8); b = _c(b, np.uint8); b_sf = _c(b_sf, np.uint8)
    nb = b.size // (K // 2)
    y = np.empty(nb)
    s = np.empty(nb)
    lib.orc_nvfp4_row_dot(_p(a), _p(a_sf), int(a_row), _p(b), _p(b_sf), nb, K, float(alpha), _p(y), _p(s))
    return y, s


def gemm_nvfp4_rows(a, a_sf, rows, b, b_sf, K, alpha=1.0):
    """Rows ``rows`` of an NVFP4 A ([rows, K] codes/scales) against every row of B:
    y[m, n] = alpha * sum_k dec(A)[rows[m], k] * dec(B)[n, k] and s the same sum of
    |terms|, both fp64 [len(rows), nb]; the same sums as nvfp4_row_dot row by row."""
    lib = _lib()
    a = _c(a, np.uint8); a_sf = _c(a_sf, np.uint8); b = _c(b, np.uint8); b_sf = _c(b_sf, np.uint8)
    r = _c(rows, np.int32)
    nb = b.size // (K // 2)
    y = np.empty((len(r), nb))
    s = np.empty((len(r), nb))
    if len(r):
        lib.orc_gemm_nvfp4_rows(_p(a), _p(a_sf), _p(r), len(r), _p(b), _p(b_sf), nb, K, float(alpha),
                                _p(y), _p(s))
    return y, s


def gemm_fp8_block(qa, sa, qb, sb, rows=None):
    """FP8 1x128-activation / 128x128-weight block-scaled GEMM in fp64.
    qa [Ma, K] uint8 e4m3, sa [Ma, K/128] f32, qb [N, K], sb [N/128, K/128];
    rows selects which A rows to evaluate (default all).  Returns (y, s) [len(rows), N]."""
    lib = _lib()
    qa = _c(qa, np.uint8); sa = _c(sa, np.float32); qb = _c(qb, np.uint8); sb = _c(sb, np.float32)
    N, K = qb.shape
    r = None if rows is None else _c(rows, np.int32)
    M = qa.shape[0] if r is None else len(r)
    y = np.empty((M, N))
    s = np.empty((M, N))
    lib.orc_gemm_fp8_block(_p(qa), _p(sa), _p(r), M, _p(qb), _p(sb), N, K, _p(y), _p(s))
    return y, s


def gemm_dense_fp8w(a, qb, sb):
    """Dense fp64 activations a [M, K] times FP8 128x128-block-scaled weights qb [N, K]."""
    lib = _lib()
    a = _c(a, np.float64); qb = _c(qb, np.uint8); sb = _c(sb, np.float32)
    M, K = a.shape
    N = qb.shape[0]
    y = np.empty((M, N))
    s = np.empty((M, N))
    lib.orc_gemm_dense_fp8w(_p(a), M, _p(qb), _p(sb), N, K, _p(y), _p(s))
    return y, s


def gemv_nvfp4_w4a16(x_bits, w, w_sf, g):
    """bf16 activations (bits, [M, K]) times NVFP4 weights (codes [N, K/2], scales
    [N, K/16]) with W's global scale g: y[m, n] = g * sum_k x[m, k] * dec(W)[n, k] and
    s = |g| * sum_k |x * dec(W)|, both fp64 [M, N]."""
    lib = _lib()
    x_bits = _c(x_bits, np.uint16); w = _c(w, np.uint8); w_sf = _c(w_sf, np.uint8)
    M, K = x_bits.shape
    N = w.shape[0]
    y = np.empty((M, N))
    s = np.empty((M, N))
    lib.orc_gemv_nvfp4_w4a16(_p(x_bits), M, _p(w), _p(w_sf), N, K, float(g), _p(y), _p(s))
    return y, s


# ----------------------------------------------------------------------------- quantizer
def quantize_nvfp4(x, g):
    """NVFP4-quantize fp32 rows x [rows, K] with global dequant scale g (fp32).
    Returns codes uint8 [rows, K/2], scales uint8 [rows, K/16]."""
    lib = _lib()
    x = _c(x, np.float32)
    rows = x.size // x.shape[-1]
    K = x.shape[-1]
    codes = np.empty(x.shape[:-1] + (K // 2,), np.uint8)
    sf = np.empty(x.shape[:-1] + (K // 16,), np.uint8)
    lib.orc_quantize_nvfp4(_p(x), rows, K, float(np.float32(g)), _p(codes), _p(sf))
    return codes, sf


# ----------------------------------------------------------------------------- routing
def route_noaux(logits, bias, n_group, topk_group, top_k, rsf):
    lib = _lib()
    assert top_k <= 64
    logits = _c(logits, np.float32); bias = _c(bias, np.float32)
    T, E = logits.shape
    ids = np.empty((T, top_k), np.int32)
    w = np.empty((T, top_k), np.float32)
    lib.orc_route_noaux(_p(logits), _p(bias), T, E, n_group, topk_group, top_k, float(rsf), _p(ids), _p(w))
    return ids, w


def dispatch(ids, E, max_m):
    lib = _lib()
    ids = _c(ids, np.int32)
    T, k = ids.shape
    masked_m = np.empty(E, np.int32)
    row = np.empty((T, k), np.int32)
    lib.orc_dispatch(_p(ids), T, E, k, max_m, _p(masked_m), _p(row))
    return masked_m, row


def dispatch_contiguous(ids, E, align):
    """Contiguous layout: counts per expert, starts = exclusive sum of the counts rounded up
    to a multiple of align ([E + 1], the last the total rows), absolute rows of the slots
    (the expert's start plus the slot's rank in token order, from dispatch)."""
    ids = _c(ids, np.int32)
    T, k = ids.shape
    count, rank = dispatch(ids, E, T * k + 1)
    padded = (count.astype(np.int64) + align - 1) // align * align
    start = np.zeros(E + 1, np.int64)
    start[1:] = np.cumsum(padded)
    return start.astype(np.int32), count, (start[ids] + rank).astype(np.int32)


def swiglu(gate_up, I):
    lib = _lib()
    gu = _c(gate_up, np.float64)
    rows = gu.size // (2 * I)
    h = np.empty(gu.shape[:-1] + (I,))
    lib.orc_swiglu(_p(gu), rows, I, _p(h))
    return h


def combine(o, s_o, w):
    """Weighted combine of one token: y* = sum_j w_j * o_j (fp64), S = sum_j |w_j| * S_j.
    o, s_o: [top_k, H]; w: [top_k]."""
    w = np.asarray(w, np.float64)[:, None]
    return (w * o).sum(axis=0), (np.abs(w) * s_o).sum(axis=0)


def num_threads() -> int:
    return int(_lib().orc_num_threads())


# ----------------------------------------------------------------------------- MoE layer
def _expert_slots(ids, row, max_m, tokens):
    """For each expert, the (subset position, slot) pairs of the given tokens routed to it
    whose row fits the capacity, in token order."""
    sub_ids = ids[tokens]
    keep = row[tokens] < max_m
    slots = {}
    for p, j in zip(*np.nonzero(keep)):
        slots.setdefault(int(sub_ids[p, j]), []).append((int(p), int(j)))
    return slots


def _combine_tokens(o, so, w, kept):
    """y*[p] = sum over kept slots j (in slot order) of w[p, j] * o[p, j] in fp64, S likewise
    of |w| * S_o (the weighted combine of the mixture-of-experts row)."""
    n, k, H = o.shape
    ystar = np.zeros((n, H))
    S = np.zeros((n, H))
    for j in range(k):
        wj = np.where(kept[:, j], w[:, j].astype(np.float64), 0.0)[:, None]
        ystar = ystar + np.where(kept[:, j][:, None], wj * o[:, j], 0.0)
        S = S + np.where(kept[:, j][:, None], np.abs(wj) * so[:, j], 0.0)
    return ystar, S


def moe_layer_nvfp4(x, g_x, ids, w, max_m, weights, g_w13, g_w2, g_h, I, tokens=None):
    """The NVFP4 expert path of one MoE layer for the given tokens (default: all), step by
    step in the order of the mixture-of-experts row ("llm-assisted-kernel-dev" README):
    dispatch into the masked layout (capacity max_m; slots past it are dropped), NVFP4
    quantization of the token rows with g_x, GEMM1 against W13 (gate rows [0, I), up rows
    [I, 2I)) with alpha = g_w13[e] * g_x, SwiGLU in fp64, requantization of the fp32 of h*
    with g_h, GEMM2 against W2 with alpha = g_w2[e] * g_h, then the weighted combine.

    x: fp32 [T, H] (bf16 values widened); ids [T, k] int32; w [T, k] fp32; weights(e) ->
    (w13 codes [2I, H/2], w13 scales [2I, H/16], w2 codes [H, I/2], w2 scales [H, I/16]).
    Returns a dict of fp64 / integer arrays over the subset positions p (tokens[p]):
    y (bf16 bits), ystar, S [n, H]; kept [n, k]; xq/xsf; per slot h (fp64 h*), hq/hsf,
    o/so (GEMM2 fp64 outputs and their |.| sums), g1/s1 (GEMM1 outputs) [n, k, ...]."""
    ids = np.asarray(ids, np.int32)
    T, k = ids.shape
    E = len(g_w13)
    tokens = np.arange(T) if tokens is None else np.asarray(tokens)
    n = len(tokens)
    _, row = dispatch(ids, E, max_m)
    xq, xsf = quantize_nvfp4(np.asarray(x, np.float32)[tokens], g_x)
    H = xq.shape[1] * 2
    out = dict(xq=xq, xsf=xsf, kept=row[tokens] < max_m, row=row[tokens],
               g1=np.full((n, k, 2 * I), np.nan), s1=np.full((n, k, 2 * I), np.nan),
               h=np.full((n, k, I), np.nan), hq=np.zeros((n, k, I // 2), np.uint8),
               hsf=np.zeros((n, k, I // 16), np.uint8), o=np.zeros((n, k, H)), so=np.zeros((n, k, H)))
    for e, sl in sorted(_expert_slots(ids, row, max_m, tokens).items()):
        w13, w13_sf, w2, w2_sf = weights(e)
        pos = np.array([p for p, _ in sl])
        js = np.array([j for _, j in sl])
        gu, s1 = gemm_nvfp4_rows(xq, xsf, pos, w13, w13_sf, H, float(g_w13[e]) * float(g_x))
        hstar = swiglu(gu, I)
        hq, hsf = quantize_nvfp4(hstar.astype(np.float32), g_h)
        o, so = gemm_nvfp4_rows(hq, hsf, np.arange(len(sl)), w2, w2_sf, I, float(g_w2[e]) * float(g_h))
        out["g1"][pos, js], out["s1"][pos, js], out["h"][pos, js] = gu, s1, hstar
        out["hq"][pos, js], out["hsf"][pos, js] = hq, hsf
        out["o"][pos, js], out["so"][pos, js] = o, so
    out["ystar"], out["S"] = _combine_tokens(out["o"], out["so"], np.asarray(w)[tokens], out["kept"])
    out["y"] = bf16_bits(out["ystar"])
    return out


def moe_layer_fp8(xq, xs, ids, w, max_m, weights, I, tokens=None, full_precision_h=False):
    """The FP8 block-scaled expert path of one MoE layer for the given tokens (default:
    all), in the order of the mixture-of-experts row ("llm-assisted-kernel-dev" README):
    dispatch (capacity max_m), GEMM1 of the 1x128-scaled e4m3 token rows against the
    128x128-scaled W13, SwiGLU in fp64, h rounded to bf16 (the optimized kernel's BF16
    default; with full_precision_h the unrounded h* is kept, as the reference's full
    precision experts), GEMM2 against the 128x128-scaled W2, then the weighted combine.

    xq e4m3 [T, H], xs fp32 [T, H/128]; weights(e) -> (w13 [2I, H], w13 scales
    [2I/128, H/128], w2 [H, I], w2 scales [H/128, I/128]).  Returns a dict as
    moe_layer_nvfp4 (h holds h*, hb the bf16 h actually multiplied)."""
    ids = np.asarray(ids, np.int32)
    T, k = ids.shape
    tokens = np.arange(T) if tokens is None else np.asarray(tokens)
    n = len(tokens)
    H = xq.shape[1]
    E = int(ids.max()) + 1 if ids.size else 1
    _, row = dispatch(ids, max(E, 1), max_m)
    out = dict(kept=row[tokens] < max_m, row=row[tokens],
               g1=np.full((n, k, 2 * I), np.nan), s1=np.full((n, k, 2 * I), np.nan),
               h=np.full((n, k, I), np.nan), hb=np.full((n, k, I), np.nan),
               o=np.zeros((n, k, H)), so=np.zeros((n, k, H)))
    for e, sl in sorted(_expert_slots(ids, row, max_m, tokens).items()):
        w13, w13_s, w2, w2_s = weights(e)
        pos = np.array([p for p, _ in sl])
        js = np.array([j for _, j in sl])
        gu, s1 = gemm_fp8_block(xq, xs, w13, w13_s, rows=np.asarray(tokens)[pos])
        hstar = swiglu(gu, I)
        hb = hstar if full_precision_h else bf16_value(bf16_bits(hstar))
        o, so = gemm_dense_fp8w(hb, w2, w2_s)
        out["g1"][pos, js], out["s1"][pos, js], out["h"][pos, js], out["hb"][pos, js] = gu, s1, hstar, hb
        out["o"][pos, js], out["so"][pos, js] = o, so
    out["ystar"], out["S"] = _combine_tokens(out["o"], out["so"], np.asarray(w)[tokens], out["kept"])
    out["y"] = bf16_bits(out["ystar"])
    return out
