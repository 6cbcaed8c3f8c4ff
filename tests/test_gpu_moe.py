"""GPU parity of the MoE expert path (routing -> dispatch -> GEMM1 -> SwiGLU -> GEMM2 ->
combine) for the NVFP4 and the FP8 block-scaled precisions.

Each stage is checked against the oracle applied to the GPU's own inputs to that stage
(teacher forcing): a GPU that accumulates in fp32 may legitimately land on the other
side of a bf16 / e2m1 rounding boundary than the fp64 oracle, and one flipped code
changes everything downstream.  Integer stages (ids, rows, masked_m, codes, scale
bytes) are bit-exact; the timed run (no debug output) must reproduce y bit for bit.

SwiGLU tolerance (derived): with the GEMM1 outputs inside t_g = 1e-5 S_g + ulp32(g),
t_u = 1e-5 S_u + ulp32(u), and |silu'| <= 1.1,
    |h_gpu - h*| <= 1.1 (|u| + t_u) t_g + |silu(g)| t_u + 8 ulp32(h*)
(+ 1 bf16 ulp when h is stored as bf16).
"""
import numpy as np
import pytest
import torch
from scipy.special import expit

import datagen
import oracle
from _helpers import assert_within, bf16_from_bits_np, bf16_tensor_bits, log, np_, ulp_bf16, ulp_f32

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


def _swiglu_tol(g, u, Sg, Su, h):
    tg = 1e-5 * Sg + ulp_f32(g)
    tu = 1e-5 * Su + ulp_f32(u)
    return 1.1 * (np.abs(u) + tu) * tg + np.abs(g * expit(g)) * tu + 8 * ulp_f32(h)


def _tokens(T, n, seed):
    if n is None or n >= T:
        return list(range(T))
    rng = np.random.default_rng(seed)
    return sorted(rng.choice(T, size=n, replace=False).tolist())


# ----------------------------------------------------------------------------- NVFP4
def _run_nvfp4(T, H, I, seed, n_check, cap=None, n_deep=0):
    mxg = _mxg()
    wl = datagen.moe_nvfp4_workload(seed, DEV, T=T, H=H, I=I)
    t, s = wl.tensors, wl.scalars
    ids, w, masked_m, row, max_m = _route_dispatch(t, cap)
    y_dbg = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    y = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    dbg_h = torch.full((E, max_m, I), float("nan"), dtype=torch.float32, device=DEV)
    common = dict(precision=mxg.MXG_MOE_NVFP4, T=T, H=H, I=I, E=E, top_k=TOPK, max_m=max_m,
                  x=t["x"], w13=t["w13"], w13_scale=t["w13_sf"], w2=t["w2"], w2_scale=t["w2_sf"],
                  topk_ids=ids, topk_w=w, masked_m=masked_m, row=row, g_x=s["g_x"], g_w13=t["g_w13"],
                  g_w2=t["g_w2"], g_h=s["g_h"])
    d_dbg = mxg.make_moe_desc(y=y_dbg, dbg_h=dbg_h, **common)
    d = mxg.make_moe_desc(y=y, **common)
    off = mxg.moe_expert_forward_workspace_layout(d)
    ws = torch.empty((off[5],), dtype=torch.uint8, device=DEV)
    mxg.moe_expert_forward(d_dbg, ws)
    torch.cuda.synchronize()
    wsh = {"a": np_(ws[off[0]:off[0] + E * max_m * H // 2]).reshape(E, max_m, H // 2),
           "a_sf": np_(ws[off[1]:off[1] + E * max_m * H // 16]).reshape(E, max_m, H // 16),
           "hc": np_(ws[off[2]:off[2] + E * max_m * I // 2]).reshape(E, max_m, I // 2),
           "hsf": np_(ws[off[3]:off[3] + E * max_m * I // 16]).reshape(E, max_m, I // 16)}
    mxg.moe_expert_forward(d, ws)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_dbg.view(torch.int16)), "timed run differs from debug run"

    ids_h, w_h, row_h = np_(ids), np_(w), np_(row)
    dbg = np_(dbg_h)
    yb = bf16_from_bits_np(bf16_tensor_bits(y))
    xq, xsf = oracle.quantize_nvfp4(np_(t["x"].float()), s["g_x"])
    g_w13, g_w2 = np_(t["g_w13"]), np_(t["g_w2"])
    wcache = {}

    def weights(e):
        if e not in wcache:
            wcache[e] = (np_(t["w13"][e]), np_(t["w13_sf"][e]), np_(t["w2"][e]), np_(t["w2_sf"][e]))
        return wcache[e]

    toks = _tokens(T, n_check, seed)
    if n_deep:
        # tokens with a slot past the first 256 rows of its expert (a later M tile)
        deep = np.flatnonzero(((row_h >= 256) & (row_h < max_m)).any(axis=1))
        assert len(deep) >= n_deep, "workload has too few rows past 256"
        toks = sorted(set(toks) | set(deep[np.linspace(0, len(deep) - 1, n_deep).astype(int)].tolist()))
    for tt in toks:
        o_list, so_list, wj = [], [], []
        for j in range(TOPK):
            e, r = int(ids_h[tt, j]), int(row_h[tt, j])
            if r >= max_m:
                continue  # dropped by the capacity
            w13, w13sf, w2, w2sf = weights(e)
            assert np.array_equal(wsh["a"][e, r], xq[tt]) and np.array_equal(wsh["a_sf"][e, r], xsf[tt]), \
                f"quantized x token {tt} slot {j}"
            gu, S1 = oracle.nvfp4_row_dot(wsh["a"][e], wsh["a_sf"][e], r, w13, w13sf, H,
                                          float(g_w13[e]) * s["g_x"])
            g, u, Sg, Su = gu[:I], gu[I:], S1[:I], S1[I:]
            hstar = oracle.swiglu(gu[None], I)[0]
            tol = _swiglu_tol(g, u, Sg, Su, hstar)
            err = np.abs(dbg[e, r].astype(np.float64) - hstar)
            assert np.all(err <= tol), f"h token {tt} slot {j}: max excess {np.max(err - tol)}"
            hq, hs = oracle.quantize_nvfp4(dbg[e, r][None], s["g_h"])
            assert np.array_equal(wsh["hc"][e, r], hq[0]) and np.array_equal(wsh["hsf"][e, r], hs[0]), \
                f"requantized h token {tt} slot {j}"
            o, So = oracle.nvfp4_row_dot(wsh["hc"][e], wsh["hsf"][e], r, w2, w2sf, I, float(g_w2[e]) * s["g_h"])
            o_list.append(o); so_list.append(So); wj.append(w_h[tt, j])
        if not o_list:
            assert np.all(yb[tt] == 0), f"token {tt} fully dropped must give y = 0"
            continue
        ystar, S = oracle.combine(np.array(o_list), np.array(so_list), np.array(wj))
        assert_within(yb[tt], ystar, S, f"y token {tt}")
    log(f"NVFP4 MoE T={T} H={H} I={I} max_m={max_m}: {len(toks)} tokens checked, "
        f"{len(wcache)} experts touched")


def test_moe_nvfp4_small_full():
    log("NVFP4 MoE small: T=64 H=512 I=256 E=256, every token")
    _run_nvfp4(64, 512, 256, 4000, None)


def test_moe_nvfp4_decode_small_full():
    log("NVFP4 MoE decode-shaped: T=32 H=1024 I=512 (capacity <= 32), every token")
    _run_nvfp4(32, 1024, 512, 4002, None)


def test_moe_nvfp4_capacity_drop():
    log("NVFP4 MoE with a capacity below the busiest expert (slots dropped)")
    _run_nvfp4(96, 256, 128, 4001, None, cap=2)


def test_moe_nvfp4_prefill_small():
    log("NVFP4 MoE prefill, small dims: T=4096 H=512 I=256 (row capacity 240), 48 tokens")
    _run_nvfp4(4096, 512, 256, 4003, 48)


def test_moe_nvfp4_prefill_two_m_tiles():
    log("NVFP4 MoE prefill with masked_m past 256: T=8192 H=512 I=256, 24 tokens")
    _run_nvfp4(8192, 512, 256, 4004, 8, n_deep=16)


def test_moe_nvfp4_decode_full_size():
    log("NVFP4 MoE decode: T=64 H=7168 I=2048, 6 tokens checked")
    _run_nvfp4(64, 7168, 2048, 1004, 6)


def test_moe_nvfp4_prefill_full_size():
    log("NVFP4 MoE prefill: T=8192 H=7168 I=2048, 3 tokens checked")
    _run_nvfp4(8192, 7168, 2048, 1004, 3)


# ----------------------------------------------------------------------------- FP8
def _vary_block_scales(s, seed, zero_frac=0.1):
    """Input variant: each 128x128 block scale times 2^u, u uniform in [-8, 8], and about
    zero_frac of the blocks set to zero (such a block contributes nothing)."""
    g = torch.Generator().manual_seed(seed)
    f = torch.pow(2.0, torch.randint(-8, 9, tuple(s.shape), generator=g).float())
    f[torch.rand(tuple(s.shape), generator=g) < zero_frac] = 0.0
    return (s.cpu() * f).to(s.device)


def _run_fp8(T, H, I, seed, n_check, n_deep=0, vary_w2_scales=False, f32h=False):
    """FP8 layer, checked stage by stage on the GPU's own intermediates.  With f32h the
    intermediate is kept as bf16 hi and lo planes (h = hi + lo to about 16 bits): h is
    checked against the oracle's unrounded SwiGLU, GEMM2 and the combine against the
    oracle on hi + lo, and y also against the oracle's whole layer on the unrounded h
    with the h tolerance carried through GEMM2."""
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
    mxg.moe_expert_forward(d, ws)
    torch.cuda.synchronize()
    y1 = y.clone()
    mxg.moe_expert_forward(d, ws)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y1.view(torch.int16)), "two runs differ"
    a = np_(ws[off[0]:off[0] + E * max_m * H]).reshape(E, max_m, H)
    cap_s = (max_m + 3) // 4 * 4  # the row scales are stored transposed: [E, H/128, cap_s]
    a_s = np_(ws[off[1]:off[1] + E * (H // 128) * cap_s * 4].view(torch.float32)).reshape(E, H // 128, cap_s)
    a_s = np.ascontiguousarray(a_s[:, :, :max_m].transpose(0, 2, 1))
    hb = np_(ws[off[2]:off[2] + E * max_m * planes * I * 2].view(torch.int16)).view(np.uint16)
    hb = hb.reshape(E, max_m, planes * I)
    ids_h, w_h, row_h = np_(ids), np_(w), np_(row)
    xq, xs = np_(t["xq"]), np_(t["xs"])
    yb = bf16_from_bits_np(bf16_tensor_bits(y))
    toks = _tokens(T, n_check, seed)
    if n_deep:
        # tokens with a slot past the first 256 rows of its expert (a later M tile)
        deep = np.flatnonzero((row_h >= 256).any(axis=1))
        assert len(deep) >= n_deep, "workload has too few rows past 256"
        toks = sorted(set(toks) | set(deep[np.linspace(0, len(deep) - 1, n_deep).astype(int)].tolist()))
    touched = set()
    if f32h:
        o_gpu = np_(ws[off[4]:off[4] + E * max_m * H * 4].view(torch.float32)).reshape(E, max_m, H)
        err2 = {"split": 0.0, "bf16": 0.0}
    for tt in toks:
        o_list, so_list, wj = [], [], []
        ox_list, sx_list, px_list = [], [], []
        for j in range(TOPK):
            e, r = int(ids_h[tt, j]), int(row_h[tt, j])
            touched.add(e)
            assert np.array_equal(a[e, r], xq[tt]) and np.array_equal(a_s[e, r], xs[tt]), f"gathered x {tt}/{j}"
            w13, w13s = np_(t["w13"][e]), np_(t["w13_s"][e])
            gu, S1 = oracle.gemm_fp8_block(xq, xs, w13, w13s, rows=[tt])
            gu, S1 = gu[0], S1[0]
            g, u = gu[:I], gu[I:]
            hstar = oracle.swiglu(gu[None], I)[0]
            if f32h:
                tol_h = _swiglu_tol(g, u, S1[:I], S1[I:], hstar)
                tol = tol_h + 2.0 ** -17 * np.abs(hstar)
                hv = bf16_from_bits_np(hb[e, r, :I]) + bf16_from_bits_np(hb[e, r, I:])
            else:
                tol = _swiglu_tol(g, u, S1[:I], S1[I:], hstar) + ulp_bf16(hstar)
                hv = bf16_from_bits_np(hb[e, r])
            err = np.abs(hv - hstar)
            assert np.all(err <= tol), f"h token {tt} slot {j}: max excess {np.max(err - tol)}"
            o, So = oracle.gemm_dense_fp8w(hv[None], np_(t["w2"][e]), np_(t["w2_s"][e]))
            o_list.append(o[0]); so_list.append(So[0]); wj.append(w_h[tt, j])
            if f32h:
                # the whole layer on the unrounded h, and how far the GPU's h may sit from it
                ox, Sx = oracle.gemm_dense_fp8w(hstar[None], np_(t["w2"][e]), np_(t["w2_s"][e]))
                w2_abs = np_(t["w2"][e]) & 0x7F  # |W2| codes (sign bit cleared)
                px, _ = oracle.gemm_dense_fp8w(tol[None], w2_abs, np.abs(np_(t["w2_s"][e])))
                ox_list.append(ox[0]); sx_list.append(Sx[0]); px_list.append(np.abs(px[0]))
                # GEMM2's fp32 output against the unrounded h, next to what a bf16 h gives
                ob, _ = oracle.gemm_dense_fp8w(oracle.bf16_value(oracle.bf16_bits(hstar))[None], np_(t["w2"][e]),
                                               np_(t["w2_s"][e]))
                err2["split"] += float(np.sum((o_gpu[e, r] - ox[0]) ** 2))
                err2["bf16"] += float(np.sum((ob[0] - ox[0]) ** 2))
        ystar, S = oracle.combine(np.array(o_list), np.array(so_list), np.array(wj))
        assert_within(yb[tt], ystar, S, f"y token {tt}")
        if f32h:
            yx, Sxx = oracle.combine(np.array(ox_list), np.array(sx_list), np.array(wj))
            carry = np.abs(np.array(wj)) @ np.array(px_list)
            assert_within(yb[tt], yx, Sxx + carry / 1e-5, f"y token {tt} against the unrounded h")
    if f32h:
        ratio = (err2["split"] / err2["bf16"]) ** 0.5
        log(f"GEMM2 rms error against the unrounded h: hi/lo planes / bf16 h = {ratio:.4f}")
        assert ratio < 0.05, f"the hi/lo intermediate is not much closer to the unrounded h ({ratio:.3f})"
    log(f"FP8 MoE T={T} H={H} I={I} max_m={max_m}: {len(toks)} tokens, {len(touched)} experts")


def test_moe_fp8_small_full():
    log("FP8 MoE small: T=128 H=512 I=256 E=256, every token")
    _run_fp8(128, 512, 256, 3000, None)


def test_moe_fp8_wide_rows_full():
    # top-8 with H % 256 == 0: the combine runs one wave per 256 columns of a token
    log("FP8 MoE: T=128 H=1024 I=256 E=256, every token")
    _run_fp8(128, 1024, 256, 3004, None)


def test_moe_fp8_two_m_tiles():
    log("FP8 MoE with masked_m past 256: T=8192 H=512 I=256 E=256, 24 tokens")
    _run_fp8(8192, 512, 256, 3001, 8, n_deep=16)


@pytest.mark.parametrize("H", [512, 384])
def test_moe_fp8_varied_w2_scales(H):
    # GEMM2 keeps its sum in units of the current block scale: scales that jump by up to
    # 2^16 between blocks, zero blocks, and (H = 384) 128-column items
    log(f"FP8 MoE with varied W2 block scales: T=256 H={H} I=384 E=256, every token")
    _run_fp8(256, H, 384, 3002 + H, None, vary_w2_scales=True)


def test_moe_fp8_full_precision_intermediate():
    log("FP8 MoE with hi/lo bf16 intermediate: T=256 H=512 I=384 E=256, every token")
    _run_fp8(256, 512, 384, 3010, None, f32h=True)


def test_moe_fp8_full_precision_intermediate_full_size():
    log("FP8 MoE with hi/lo bf16 intermediate: T=4096 H=7168 I=2048, 3 tokens checked")
    _run_fp8(4096, 7168, 2048, 1003, 3, f32h=True)


def test_moe_fp8_full_size():
    log("FP8 MoE prefill: T=4096 H=7168 I=2048, 3 tokens checked")
    _run_fp8(4096, 7168, 2048, 1003, 3)
