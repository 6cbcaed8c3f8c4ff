"""GPU parity of the MoE expert path (routing -> dispatch -> GEMM1 -> SwiGLU -> GEMM2 ->
combine) for the NVFP4 and the FP8 block-scaled precisions.

Routing and dispatch are bit-exact against the oracle over every token.  The expert
stages are checked per expert on a token subset (every token at reduced sizes, 512
tokens plus rows past the first 256-row M tile at the full prefill sizes, every token of
the full decode batch), each stage against the oracle applied to the GPU's own inputs
(tests/_moe_check.py).  The timed run (no debug output) must reproduce y bit for bit.
"""
import numpy as np
import pytest
import torch

import datagen
import oracle
from _helpers import bf16_tensor_bits, log, np_
from _moe_check import check_fp8_layer, check_nvfp4_layer, tokens_subset

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0") if torch.cuda.is_available() else None
E, TOPK = 256, 8


def _mxg():
    import fp8_grouped_gemm_nvfp4_amd as mxg
    return mxg


def _route_dispatch(t, cap=None):
    mxg = _mxg()
    ids, w = mxg.moe_route_noaux(t["logits"], t["bias"], 8, 4, TOPK, 2.5)
    if cap is None:
        mm_full, _ = mxg.moe_dispatch(ids, E, 1 << 20)
        cap = max(16, -(-int(mm_full.max().item()) // 16) * 16)
    masked_m, row = mxg.moe_dispatch(ids, E, cap)
    torch.cuda.synchronize()
    ids_o, w_o = oracle.route_noaux(np_(t["logits"]), np_(t["bias"]), 8, 4, TOPK, 2.5)
    assert np.array_equal(np_(ids), ids_o), "routing ids"
    assert np.array_equal(np_(w).view(np.uint32), w_o.view(np.uint32)), "routing weights"
    mm_o, row_o = oracle.dispatch(ids_o, E, cap)
    assert np.array_equal(np_(masked_m), mm_o) and np.array_equal(np_(row), row_o), "dispatch"
    return ids, w, masked_m, row, cap


def _region(ws, off, i, shape, dtype=torch.uint8):
    """Per-expert view e -> numpy array of workspace region i laid out as [E, *shape]."""
    n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()

    def get(e):
        b = ws[off[i] + e * n: off[i] + (e + 1) * n]
        return np_(b.view(dtype)).reshape(shape)
    return get


def _cached(fn):
    cache = {}

    def get(e):
        if e not in cache:
            cache[e] = fn(e)
        return cache[e]
    return get


# ----------------------------------------------------------------------------- NVFP4
def _run_nvfp4(T, H, I, seed, n_check, cap=None, n_deep=0, e2e=0, report_h_scales=False):
    mxg = _mxg()
    wl = datagen.moe_nvfp4_workload(seed, DEV, T=T, H=H, I=I)
    t, s = wl.tensors, wl.scalars
    ids, w, masked_m, row, max_m = _route_dispatch(t, cap)
    y_dbg = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    y = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    dbg_h = torch.full((E, max_m, I), float("nan"), dtype=torch.float32, device=DEV)
    dbg_g1 = torch.full((E, max_m, 2 * I), float("nan"), dtype=torch.float32, device=DEV)
    common = dict(precision=mxg.MXG_MOE_NVFP4, T=T, H=H, I=I, E=E, top_k=TOPK, max_m=max_m,
                  x=t["x"], w13=t["w13"], w13_scale=t["w13_sf"], w2=t["w2"], w2_scale=t["w2_sf"],
                  topk_ids=ids, topk_w=w, masked_m=masked_m, row=row, g_x=s["g_x"], g_w13=t["g_w13"],
                  g_w2=t["g_w2"], g_h=s["g_h"])
    d_dbg = mxg.make_moe_desc(y=y_dbg, dbg_h=dbg_h, dbg_g1=dbg_g1, **common)
    d = mxg.make_moe_desc(y=y, **common)
    off = mxg.moe_expert_forward_workspace_layout(d)
    ws = torch.empty((off[5],), dtype=torch.uint8, device=DEV)
    mxg.moe_expert_forward(d_dbg, ws)
    torch.cuda.synchronize()
    ws_dbg = ws.clone()
    mxg.moe_expert_forward(d, ws)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_dbg.view(torch.int16)), "timed run differs from debug run"
    ids_h, row_h = np_(ids), np_(row)
    ga = _region(ws_dbg, off, 0, (max_m, H // 2)); gs = _region(ws_dbg, off, 1, (max_m, H // 16))
    hc = _region(ws_dbg, off, 2, (max_m, I // 2)); hs = _region(ws_dbg, off, 3, (max_m, I // 16))
    if report_h_scales:
        mm = np_(masked_m)
        valid = torch.arange(max_m, device=DEV)[None, :] < masked_m[:, None]
        hsf = ws_dbg[off[3]:off[3] + E * max_m * (I // 16)].view(E, max_m, I // 16)[valid]
        n_blk = hsf.numel()
        sat = int((hsf == 0x7E).sum().item()); zero = int((hsf == 0).sum().item())
        log(f"NVFP4 h block scales with g_h = {s['g_h']}: {n_blk} blocks over {int(mm.sum())} valid rows, "
            f"{sat} at 448 ({sat / n_blk:.2e}), {zero} zero ({zero / n_blk:.2e}); "
            f"largest scale code 0x{int(hsf.max().item()):02X}")
    toks = tokens_subset(T, n_check, seed, row_h, max_m, n_deep)
    log(f"NVFP4 MoE T={T} H={H} I={I} max_m={max_m}: checking {len(toks)} tokens")
    check_nvfp4_layer(
        x=np_(t["x"].float()), g_x=s["g_x"], ids=ids_h, w=np_(w), row=row_h, max_m=max_m, I=I,
        weights=_cached(lambda e: (np_(t["w13"][e]), np_(t["w13_sf"][e]), np_(t["w2"][e]), np_(t["w2_sf"][e]))),
        g_w13=np_(t["g_w13"]), g_w2=np_(t["g_w2"]), g_h=s["g_h"],
        gathered=lambda e: (ga(e), gs(e), hc(e), hs(e)), h_pre=lambda e: np_(dbg_h[e]),
        y_bits=bf16_tensor_bits(y), toks=toks, what=f"NVFP4 T={T} H={H}", e2e_tokens=e2e,
        g1=lambda e: np_(dbg_g1[e]))


def test_moe_nvfp4_small_full():
    log("NVFP4 MoE small: T=64 H=512 I=256 E=256, every token")
    _run_nvfp4(64, 512, 256, 4000, None, e2e=64)


def test_moe_nvfp4_decode_small_full():
    log("NVFP4 MoE decode-shaped: T=32 H=1024 I=512 (capacity <= 32), every token")
    _run_nvfp4(32, 1024, 512, 4002, None, e2e=32)


def test_moe_nvfp4_capacity_drop():
    log("NVFP4 MoE with a capacity below the busiest expert (slots dropped)")
    _run_nvfp4(96, 256, 128, 4001, None, cap=2, e2e=96)


def test_moe_nvfp4_prefill_small():
    log("NVFP4 MoE prefill, small dims: T=4096 H=512 I=256 (row capacity 240), 512 tokens")
    _run_nvfp4(4096, 512, 256, 4003, 512, e2e=64)


def test_moe_nvfp4_prefill_two_m_tiles():
    log("NVFP4 MoE prefill with masked_m past 256: T=8192 H=512 I=256, 512 tokens + 64 past row 256")
    _run_nvfp4(8192, 512, 256, 4004, 512, n_deep=64)


def test_moe_nvfp4_decode_full_size():
    log("NVFP4 MoE decode: T=64 H=7168 I=2048, every token")
    _run_nvfp4(64, 7168, 2048, 1004, None, e2e=8, report_h_scales=True)


def test_moe_nvfp4_prefill_full_size():
    log("NVFP4 MoE prefill: T=8192 H=7168 I=2048, 512 tokens + 32 past row 256")
    _run_nvfp4(8192, 7168, 2048, 1004, 512, n_deep=32, e2e=4, report_h_scales=True)


# ----------------------------------------------------------------------------- FP8
def _vary_block_scales(s, seed, zero_frac=0.1):
    """Input variant: each 128x128 block scale times 2^u, u uniform in [-8, 8], and about
    zero_frac of the blocks set to zero (such a block contributes nothing)."""
    g = torch.Generator().manual_seed(seed)
    f = torch.pow(2.0, torch.randint(-8, 9, tuple(s.shape), generator=g).float())
    f[torch.rand(tuple(s.shape), generator=g) < zero_frac] = 0.0
    return (s.cpu() * f).to(s.device)


def _run_fp8(T, H, I, seed, n_check, n_deep=0, vary_w2_scales=False, f32h=False, e2e=0):
    mxg = _mxg()
    prec = mxg.MXG_MOE_FP8_BLOCK128_F32H if f32h else mxg.MXG_MOE_FP8_BLOCK128
    planes = 2 if f32h else 1
    wl = datagen.moe_fp8_workload(seed, DEV, T=T, H=H, I=I)
    t = wl.tensors
    if vary_w2_scales:
        t["w2_s"] = _vary_block_scales(t["w2_s"], seed + 1)
    ids, w, masked_m, row, max_m = _route_dispatch(t)
    y = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    d = mxg.make_moe_desc(prec, T, H, I, E, TOPK, max_m, t["xq"], t["w13"], t["w13_s"],
                          t["w2"], t["w2_s"], ids, w, masked_m, row, y, x_scale=t["xs"])
    off = mxg.moe_expert_forward_workspace_layout(d)
    ws = torch.empty((off[5],), dtype=torch.uint8, device=DEV)
    dbg_g1 = torch.full((E, max_m, 2 * I), float("nan"), dtype=torch.float32, device=DEV)
    y_dbg = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    d_dbg = mxg.make_moe_desc(prec, T, H, I, E, TOPK, max_m, t["xq"], t["w13"], t["w13_s"],
                              t["w2"], t["w2_s"], ids, w, masked_m, row, y_dbg, x_scale=t["xs"], dbg_g1=dbg_g1)
    mxg.moe_expert_forward(d_dbg, ws)
    mxg.moe_expert_forward(d, ws)
    torch.cuda.synchronize()
    y1 = y.clone()
    mxg.moe_expert_forward(d, ws)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y1.view(torch.int16)), "two runs differ"
    assert torch.equal(y.view(torch.int16), y_dbg.view(torch.int16)), "timed run differs from debug run"
    cap_s = (max_m + 3) // 4 * 4  # the row scales are stored transposed: [E, H/128, cap_s]
    gtok = _region(ws, off, 0, (max_m,), torch.int32)
    gs_t = _region(ws, off, 1, (H // 128, cap_s), torch.float32)
    hp = _region(ws, off, 2, (max_m, planes * I), torch.int16)
    og = _region(ws, off, 4, (max_m, H), torch.float32)
    row_h = np_(row)
    toks = tokens_subset(T, n_check, seed, row_h, max_m, n_deep)
    log(f"FP8 MoE T={T} H={H} I={I} max_m={max_m}: checking {len(toks)} tokens")
    check_fp8_layer(
        xq=np_(t["xq"]), xs=np_(t["xs"]), ids=np_(ids), w=np_(w), row=row_h, max_m=max_m, I=I,
        weights=_cached(lambda e: (np_(t["w13"][e]), np_(t["w13_s"][e]), np_(t["w2"][e]), np_(t["w2_s"][e]))),
        gathered=lambda e: (gtok(e), np.ascontiguousarray(gs_t(e)[:, :max_m].T)),
        h_planes=lambda e: hp(e).view(np.uint16), y_bits=bf16_tensor_bits(y), toks=toks,
        what=f"FP8{' hi/lo h' if f32h else ''} T={T} H={H}", f32h=f32h, o_gpu=og, e2e_tokens=e2e,
        g1=lambda e: np_(dbg_g1[e]))


def test_moe_fp8_small_full():
    log("FP8 MoE small: T=128 H=512 I=256 E=256, every token")
    _run_fp8(128, 512, 256, 3000, None, e2e=128)


def test_moe_fp8_wide_rows_full():
    # top-8 with H % 256 == 0: the combine runs one wave per 256 columns of a token
    log("FP8 MoE: T=128 H=1024 I=256 E=256, every token")
    _run_fp8(128, 1024, 256, 3004, None)


def test_moe_fp8_two_m_tiles():
    log("FP8 MoE with masked_m past 256: T=8192 H=512 I=256 E=256, 512 tokens + 64 past row 256")
    _run_fp8(8192, 512, 256, 3001, 512, n_deep=64)


@pytest.mark.parametrize("H", [512, 384])
def test_moe_fp8_varied_w2_scales(H):
    # GEMM2 keeps its sum in units of the current block scale: scales that jump by up to
    # 2^16 between blocks, zero blocks, and (H = 384) 128-column items
    log(f"FP8 MoE with varied W2 block scales: T=256 H={H} I=384 E=256, every token")
    _run_fp8(256, H, 384, 3002 + H, None, vary_w2_scales=True)


@pytest.mark.parametrize("H,I,f32h", [(128, 128, False), (256, 128, False), (128, 256, True)])
def test_moe_fp8_short_items(H, I, f32h):
    # GEMM1 items of one or two 128-K steps: its activation ring runs two steps ahead, so
    # its DMAs cross one or two item boundaries; GEMM2 items of two to four 64-K steps
    log(f"FP8 MoE with short items: T=256 H={H} I={I} E=256{' hi/lo h' if f32h else ''}, every token")
    _run_fp8(256, H, I, 3020 + H + I, None, f32h=f32h)


def test_moe_fp8_full_precision_intermediate():
    log("FP8 MoE with hi/lo bf16 intermediate: T=256 H=512 I=384 E=256, every token")
    _run_fp8(256, 512, 384, 3010, None, f32h=True, e2e=64)


def test_moe_fp8_full_precision_intermediate_full_size():
    log("FP8 MoE with hi/lo bf16 intermediate: T=4096 H=7168 I=2048, 64 tokens")
    _run_fp8(4096, 7168, 2048, 1003, 64, f32h=True)


def test_moe_fp8_full_size():
    log("FP8 MoE prefill: T=4096 H=7168 I=2048, 512 tokens")
    _run_fp8(4096, 7168, 2048, 1003, 512, e2e=4)
