"""C-ABI checks that need no GPU: the library loads, exports every symbol the header
declares, and rejects bad arguments with the documented status before any HIP call."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxg.h")

import fp8_grouped_gemm_nvfp4_amd as mxg  # noqa: E402

if not os.path.exists(mxg.LIB_PATH):
    from fp8_grouped_gemm_nvfp4_amd import _build
    _build.build()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?(?:int|size_t|char\s*\*|const char\s*\*)\s*\*?\s*(\w+)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


def test_header_lists_entry_points():
    names = _declared_functions()
    for want in ["mx_grouped_gemm_masked", "mx_grouped_gemm", "mx_grouped_gemm_contiguous", "moe_dispatch_contiguous",
                 "mx_gemv_nvfp4_w4a16", "mx_quantize_nvfp4", "moe_route_noaux",
                 "moe_dispatch", "moe_quantize_gather_nvfp4", "moe_expert_forward",
                 "moe_expert_forward_workspace_size", "moe_expert_forward_workspace_layout",
                 "mxg_status_string", "mxg_last_error", "mxg_version"]:
        assert want in names, want


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(mxg.LIB_PATH)
    for name in _declared_functions():
        assert hasattr(lib, name), name
    # the binding declares a signature for each of them
    assert set(_declared_functions()) <= set(mxg.SIGNATURES)


def test_status_strings():
    L = mxg.lib()
    for code, name in enumerate(["MXG_OK", "MXG_ERR_INVALID_ARG", "MXG_ERR_UNSUPPORTED",
                                 "MXG_ERR_WORKSPACE", "MXG_ERR_HIP"]):
        assert L.mxg_status_string(code).decode() == name
    assert L.mxg_status_string(99).decode() == "unknown status"
    assert L.mxg_version() >= 100


P = ctypes.c_void_p
FAKE = P(1 << 20)  # never dereferenced: every call below fails validation first


def _masked(**kw):
    args = dict(a=FAKE, a_sf=FAKE, b=FAKE, b_sf=FAKE, alpha=None, masked_m=FAKE, out=FAKE, G=4,
                max_m=64, N=512, K=1024, ab=mxg.MXG_E2M1, sf=mxg.MXG_E4M3, c=mxg.MXG_BF16, vec=16,
                cu=0, stream=None)
    args.update(kw)
    return mxg.lib().mx_grouped_gemm_masked(*args.values())


@pytest.mark.parametrize("kw,status", [
    (dict(a=None), mxg.MXG_ERR_INVALID_ARG),
    (dict(masked_m=None), mxg.MXG_ERR_INVALID_ARG),
    (dict(G=0), mxg.MXG_ERR_INVALID_ARG),
    (dict(max_m=0), mxg.MXG_ERR_INVALID_ARG),
    (dict(N=-1), mxg.MXG_ERR_INVALID_ARG),
    (dict(K=1000), mxg.MXG_ERR_UNSUPPORTED),
    (dict(ab=mxg.MXG_E4M3), mxg.MXG_ERR_UNSUPPORTED),
    (dict(vec=32), mxg.MXG_ERR_UNSUPPORTED),
    (dict(c=mxg.MXG_E2M1), mxg.MXG_ERR_UNSUPPORTED),
    (dict(cu=-1), mxg.MXG_ERR_INVALID_ARG),
    (dict(a=P((1 << 20) + 8)), mxg.MXG_ERR_INVALID_ARG),
])
def test_masked_gemm_rejects(kw, status):
    assert _masked(**kw) == status
    assert mxg.lib().mxg_last_error().decode() != ""


def test_hetero_rejects():
    L = mxg.lib()
    arr = (mxg.GroupDesc * 2)()
    arr[0] = mxg.GroupDesc(128, 256, 1024, 0, 1.0, FAKE, FAKE, FAKE, FAKE, FAKE)
    arr[1] = mxg.GroupDesc(16, 256, 1000, 0, 1.0, FAKE, FAKE, FAKE, FAKE, FAKE)
    assert L.mx_grouped_gemm(arr, 2, 1, 2, 3, 16, 0, None) == mxg.MXG_ERR_UNSUPPORTED
    assert L.mx_grouped_gemm(arr, 0, 1, 2, 3, 16, 0, None) == mxg.MXG_ERR_INVALID_ARG
    assert L.mx_grouped_gemm(arr, 33, 1, 2, 3, 16, 0, None) == mxg.MXG_ERR_INVALID_ARG
    arr[1] = mxg.GroupDesc(16, 256, 1024, 100, 1.0, FAKE, FAKE, FAKE, FAKE, FAKE)
    assert L.mx_grouped_gemm(arr, 2, 1, 2, 3, 16, 0, None) == mxg.MXG_ERR_INVALID_ARG  # ldc < N
    assert L.mx_grouped_gemm(None, 1, 1, 2, 3, 16, 0, None) == mxg.MXG_ERR_INVALID_ARG


def test_gemv_w4a16_rejects():
    L = mxg.lib()
    args = dict(x=FAKE, M=1, K=4096, w=FAKE, w_sf=FAKE, g=0.5, out=FAKE, N=4096, c=mxg.MXG_BF16, cu=0, s=None)
    for kw, status in [(dict(x=None), mxg.MXG_ERR_INVALID_ARG), (dict(M=0), mxg.MXG_ERR_INVALID_ARG),
                       (dict(N=0), mxg.MXG_ERR_INVALID_ARG), (dict(M=5), mxg.MXG_ERR_UNSUPPORTED),
                       (dict(K=4000), mxg.MXG_ERR_UNSUPPORTED), (dict(M=3, K=16384), mxg.MXG_ERR_UNSUPPORTED),
                       (dict(c=mxg.MXG_E2M1), mxg.MXG_ERR_UNSUPPORTED), (dict(cu=-1), mxg.MXG_ERR_INVALID_ARG),
                       (dict(out=P((1 << 20) + 4)), mxg.MXG_ERR_INVALID_ARG)]:
        a = dict(args, **kw)
        assert L.mx_gemv_nvfp4_w4a16(*a.values()) == status, kw
        assert L.mxg_last_error().decode() != ""


def test_contiguous_rejects():
    L = mxg.lib()
    args = dict(a=FAKE, a_sf=FAKE, b=FAKE, b_sf=FAKE, alpha=None, gs=FAKE, cnt=FAKE, out=FAKE, G=8, M=4096, N=512,
                K=1024, ab=mxg.MXG_E2M1, sf=mxg.MXG_E4M3, c=mxg.MXG_BF16, vec=16, cu=0, s=None)
    for kw, status in [(dict(gs=None), mxg.MXG_ERR_INVALID_ARG), (dict(G=0), mxg.MXG_ERR_INVALID_ARG),
                       (dict(M=0), mxg.MXG_ERR_INVALID_ARG), (dict(G=513), mxg.MXG_ERR_UNSUPPORTED),
                       (dict(N=520), mxg.MXG_ERR_UNSUPPORTED), (dict(K=1088), mxg.MXG_ERR_UNSUPPORTED),
                       (dict(vec=32), mxg.MXG_ERR_UNSUPPORTED), (dict(a=P((1 << 20) + 8)), mxg.MXG_ERR_INVALID_ARG)]:
        a = dict(args, **kw)
        assert L.mx_grouped_gemm_contiguous(*a.values()) == status, kw
    assert L.moe_dispatch_contiguous(FAKE, 8, 256, 8, 0, FAKE, FAKE, FAKE, None) == mxg.MXG_ERR_INVALID_ARG
    assert L.moe_dispatch_contiguous(FAKE, 8, 256, 8, 8192, FAKE, FAKE, FAKE, None) == mxg.MXG_ERR_INVALID_ARG
    assert L.moe_dispatch_contiguous(None, 8, 256, 8, 16, FAKE, FAKE, FAKE, None) == mxg.MXG_ERR_INVALID_ARG


def test_route_dispatch_quant_reject():
    L = mxg.lib()
    assert L.moe_route_noaux(FAKE, FAKE, 8, 128, 8, 4, 8, 2.5, FAKE, FAKE, None) == mxg.MXG_ERR_UNSUPPORTED
    assert L.moe_route_noaux(FAKE, FAKE, 8, 256, 3, 2, 8, 2.5, FAKE, FAKE, None) == mxg.MXG_ERR_UNSUPPORTED
    assert L.moe_route_noaux(FAKE, FAKE, 8, 256, 8, 9, 8, 2.5, FAKE, FAKE, None) == mxg.MXG_ERR_INVALID_ARG
    assert L.moe_route_noaux(FAKE, FAKE, 8, 256, 8, 4, 9, 2.5, FAKE, FAKE, None) == mxg.MXG_ERR_UNSUPPORTED
    assert L.moe_route_noaux(None, FAKE, 8, 256, 8, 4, 8, 2.5, FAKE, FAKE, None) == mxg.MXG_ERR_INVALID_ARG
    assert L.moe_dispatch(FAKE, 8, 256, 8, 0, FAKE, FAKE, None, None) == mxg.MXG_ERR_INVALID_ARG
    assert L.moe_dispatch(None, 8, 256, 8, 8, FAKE, FAKE, FAKE, None) == mxg.MXG_ERR_INVALID_ARG
    assert L.mx_quantize_nvfp4(FAKE, mxg.MXG_BF16, 4, 24, 1.0, FAKE, FAKE, None) == mxg.MXG_ERR_UNSUPPORTED
    assert L.mx_quantize_nvfp4(FAKE, mxg.MXG_BF16, 4, 32, 0.0, FAKE, FAKE, None) == mxg.MXG_ERR_INVALID_ARG
    assert L.mx_quantize_nvfp4(FAKE, mxg.MXG_E2M1, 4, 32, 1.0, FAKE, FAKE, None) == mxg.MXG_ERR_UNSUPPORTED
    assert L.moe_quantize_gather_nvfp4(FAKE, 8, 7168, -1.0, FAKE, FAKE, 8, 256, 8, FAKE, FAKE,
                                       None) == mxg.MXG_ERR_INVALID_ARG


def _desc(**kw):
    d = mxg.MoeDesc()
    base = dict(precision=mxg.MXG_MOE_NVFP4, T=64, H=7168, I=2048, E=256, top_k=8, max_m=64,
                x=FAKE.value, x_scale=FAKE.value, g_x=0.01, w13=FAKE.value, w13_scale=FAKE.value,
                g_w13=FAKE.value, w2=FAKE.value, w2_scale=FAKE.value, g_w2=FAKE.value, g_h=1024.0,
                topk_ids=FAKE.value, topk_w=FAKE.value, masked_m=FAKE.value, row=FAKE.value,
                y=FAKE.value, dbg_h=None)
    base.update(kw)
    for k, v in base.items():
        setattr(d, k, v)
    return d


def test_moe_fp8_workspace_layout_and_expert_limit():
    L = mxg.lib()
    off = (ctypes.c_size_t * 6)()
    d = _desc(precision=mxg.MXG_MOE_FP8_BLOCK128, max_m=241)
    assert L.moe_expert_forward_workspace_layout(ctypes.byref(d), off) == mxg.MXG_OK
    rows = 256 * 241
    assert off[1] - off[0] >= rows * 4                          # the token of each expert row
    assert off[2] - off[1] >= 256 * (7168 // 128) * 244 * 4      # transposed scales, stride 244
    assert off[3] - off[2] >= (rows + 1) * 2048 * 2              # h plus the scratch row
    assert off[5] - off[4] >= rows * 7168 * 4
    d2 = _desc(precision=mxg.MXG_MOE_FP8_BLOCK128_F32H, max_m=241)
    off2 = (ctypes.c_size_t * 6)()
    assert L.moe_expert_forward_workspace_layout(ctypes.byref(d2), off2) == mxg.MXG_OK
    assert off2[3] - off2[2] >= (rows + 1) * 2 * 2048 * 2                  # hi and lo planes
    assert off2[1] - off2[0] == off[1] - off[0] and off2[2] - off2[1] == off[2] - off[1]
    for E, want in ((1024, mxg.MXG_OK), (1025, mxg.MXG_ERR_UNSUPPORTED)):
        d = _desc(precision=mxg.MXG_MOE_FP8_BLOCK128, E=E)
        assert L.moe_expert_forward_workspace_layout(ctypes.byref(d), off) == want, E
    # an expert's h rows (4 * max_m * I bytes with both planes) and the token rows of x
    # (T * H bytes) stay below 2^32
    for mm, want in ((524287, mxg.MXG_OK), (524288, mxg.MXG_ERR_UNSUPPORTED)):
        for prec in (mxg.MXG_MOE_FP8_BLOCK128, mxg.MXG_MOE_FP8_BLOCK128_F32H):
            d = _desc(precision=prec, max_m=mm)
            assert L.moe_expert_forward_workspace_layout(ctypes.byref(d), off) == want, (mm, prec)
    for T, want in ((599186, mxg.MXG_OK), (599187, mxg.MXG_ERR_UNSUPPORTED)):  # 2^32 / 7168 = 599186.3
        d = _desc(precision=mxg.MXG_MOE_FP8_BLOCK128, T=T)
        assert L.moe_expert_forward_workspace_layout(ctypes.byref(d), off) == want, T


def test_moe_workspace_layout_and_rejects():
    L = mxg.lib()
    d = _desc()
    off = (ctypes.c_size_t * 6)()
    assert L.moe_expert_forward_workspace_layout(ctypes.byref(d), off) == mxg.MXG_OK
    rows = 256 * 64
    assert off[1] >= rows * 7168 // 2 and off[5] == L.moe_expert_forward_workspace_size(ctypes.byref(d))
    assert off[5] >= rows * 7168 * 4 + rows * (7168 // 2 + 7168 // 16 + 2048 // 2 + 2048 // 16)
    assert all(o % 256 == 0 for o in off)
    # workspace too small -> MXG_ERR_WORKSPACE without touching the GPU
    assert L.moe_expert_forward(ctypes.byref(d), FAKE, 1024, None) == mxg.MXG_ERR_WORKSPACE
    assert L.moe_expert_forward(ctypes.byref(d), None, 1 << 40, None) == mxg.MXG_ERR_WORKSPACE
    for bad in [dict(precision=7), dict(H=100), dict(top_k=9), dict(g_h=0.0), dict(y=None), dict(T=-1)]:
        db = _desc(**bad)
        st = L.moe_expert_forward(ctypes.byref(db), FAKE, 1 << 40, None)
        assert st in (mxg.MXG_ERR_INVALID_ARG, mxg.MXG_ERR_UNSUPPORTED), bad
        assert L.moe_expert_forward_workspace_size(ctypes.byref(db)) == 0
    d8 = _desc(precision=mxg.MXG_MOE_FP8_BLOCK128, x_scale=None)
    assert L.moe_expert_forward(ctypes.byref(d8), FAKE, 1 << 40, None) == mxg.MXG_ERR_INVALID_ARG


def test_w13_layout_rejects():
    L = mxg.lib()
    off = (ctypes.c_size_t * 6)()
    d = _desc(w13_layout=mxg.MXG_W13_INTERLEAVED16)
    assert L.moe_expert_forward_workspace_layout(ctypes.byref(d), off) == mxg.MXG_OK
    for bad, want in [(dict(w13_layout=8), mxg.MXG_ERR_INVALID_ARG),
                      (dict(w13_layout=mxg.MXG_W13_INTERLEAVED16, precision=mxg.MXG_MOE_FP8_BLOCK128),
                       mxg.MXG_ERR_UNSUPPORTED),
                      (dict(w13_layout=mxg.MXG_W13_INTERLEAVED16, precision=mxg.MXG_MOE_FP8_BLOCK128_F32H),
                       mxg.MXG_ERR_UNSUPPORTED)]:
        db = _desc(**bad)
        assert L.moe_expert_forward(ctypes.byref(db), FAKE, 1 << 40, None) == want, bad
    # the weight re-layout: null, sizes, alignment and overlap are refused before any launch
    A, B = P(1 << 20), P(1 << 30)
    assert L.moe_interleave_w13(None, B, 4, 64, 512, None) == mxg.MXG_ERR_INVALID_ARG
    assert L.moe_interleave_w13(A, B, 4, 24, 512, None) == mxg.MXG_ERR_UNSUPPORTED   # I % 16
    assert L.moe_interleave_w13(A, B, 4, 64, 510, None) == mxg.MXG_ERR_UNSUPPORTED   # row_bytes % 4
    assert L.moe_interleave_w13(P((1 << 20) + 2), B, 4, 64, 512, None) == mxg.MXG_ERR_INVALID_ARG
    assert L.moe_interleave_w13(A, P((1 << 20) + 4096), 4, 64, 512, None) == mxg.MXG_ERR_INVALID_ARG
    assert L.moe_interleave_w13(A, B, -1, 64, 512, None) == mxg.MXG_ERR_INVALID_ARG


def test_dispatch_quantize_gather_rejects():
    L = mxg.lib()
    f = L.moe_dispatch_quantize_gather_nvfp4
    args = [FAKE, 8, 7168, 0.01, FAKE, 8, 256, 8, FAKE, FAKE, FAKE, FAKE, None]
    for i, v, want in [(0, None, mxg.MXG_ERR_INVALID_ARG), (1, -1, mxg.MXG_ERR_INVALID_ARG),
                       (2, 7168 + 32, mxg.MXG_ERR_UNSUPPORTED), (3, 0.0, mxg.MXG_ERR_INVALID_ARG),
                       (5, 0, mxg.MXG_ERR_INVALID_ARG), (7, 0, mxg.MXG_ERR_INVALID_ARG),
                       (10, P((1 << 20) + 4), mxg.MXG_ERR_INVALID_ARG)]:
        a = list(args)
        a[i] = v
        assert f(*a) == want, (i, v)


def test_product_path_fails_loudly_without_library(tmp_path, monkeypatch):
    monkeypatch.setattr(mxg, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(mxg, "_LIB", None)
    with pytest.raises(ImportError):
        mxg.lib()
