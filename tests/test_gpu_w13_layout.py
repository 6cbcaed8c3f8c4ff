"""Gate/up-interleaved W13 (MXG_W13_INTERLEAVED16) for the NVFP4 MoE layer.

The interleaved layout holds the same logical weights as the stacked one, so the layer
must give the same y bit for bit: each output's products are summed in the same order,
only the rows the kernels fetch move.  The stacked path itself is checked against the
oracle in test_gpu_moe.py.  The interleaved copies here are built with torch indexing
from a permutation written out below, independently of the library's re-layout, which is
checked against the same permutation.  Covered: the decode kernel (max_m <= 32), the
streaming kernel (larger groups) and the tiled kernel (more than 1024 experts).
"""
import numpy as np
import pytest
import torch

import datagen
from _helpers import log

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0") if torch.cuda.is_available() else None
TOPK = 8


def _mxg():
    import fp8_grouped_gemm_nvfp4_amd as mxg
    return mxg


def _perm(I):
    """Interleaved row r holds logical row perm[r]: rows [32 j, 32 j + 16) gate rows
    [16 j, 16 j + 16), rows [32 j + 16, 32 j + 32) the up rows I + 16 j + ..."""
    p = np.empty(2 * I, dtype=np.int64)
    for r in range(2 * I):
        j, w = divmod(r, 32)
        p[r] = 16 * j + w if w < 16 else I + 16 * j + (w - 16)
    assert sorted(p.tolist()) == list(range(2 * I))
    return torch.from_numpy(p).to(DEV)


@pytest.mark.parametrize("row_bytes", [64, 8, 448])
def test_interleave_w13_matches_permutation(row_bytes):
    mxg = _mxg()
    E, I = 3, 96
    g = torch.Generator(device=DEV).manual_seed(7 + row_bytes)
    src = torch.randint(0, 256, (E, 2 * I, row_bytes), dtype=torch.uint8, device=DEV, generator=g)
    got = mxg.moe_interleave_w13(src)
    torch.cuda.synchronize()
    assert torch.equal(got, src[:, _perm(I), :])


def _layer(wl, T, H, I, E, ids, w, cap, w13, w13_sf, layout):
    mxg = _mxg()
    t, s = wl.tensors, wl.scalars
    masked_m, row = mxg.moe_dispatch(ids, E, cap)
    y = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    d = mxg.make_moe_desc(mxg.MXG_MOE_NVFP4, T, H, I, E, TOPK, cap, t["x"], w13, w13_sf, t["w2"], t["w2_sf"],
                          ids, w, masked_m, row, y, g_x=s["g_x"], g_w13=t["g_w13"], g_w2=t["g_w2"],
                          g_h=s["g_h"], w13_layout=layout)
    ws = torch.empty((mxg.moe_expert_forward_workspace_size(d),), dtype=torch.uint8, device=DEV)
    mxg.moe_expert_forward(d, ws)
    torch.cuda.synchronize()
    return y, masked_m


def _check(wl, T, H, I, E, ids, w, cap, what):
    mxg = _mxg()
    t = wl.tensors
    y0, mm = _layer(wl, T, H, I, E, ids, w, cap, t["w13"], t["w13_sf"], mxg.MXG_W13_STACKED)
    p = _perm(I)
    w13_il, sf_il = t["w13"][:, p, :].contiguous(), t["w13_sf"][:, p, :].contiguous()
    y1, _ = _layer(wl, T, H, I, E, ids, w, cap, w13_il, sf_il, mxg.MXG_W13_INTERLEAVED16)
    log(f"{what}: max masked_m {int(mm.max().item())}, {int((mm > 0).sum().item())} active experts")
    assert not torch.isnan(y0.float()).any()
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16)), f"{what}: interleaved y differs"


@pytest.mark.parametrize("T,what", [(16, "decode kernel"), (512, "streaming kernel")])
def test_moe_nvfp4_interleaved_w13_bit_identical(T, what):
    mxg = _mxg()
    E, H, I = 256, 512, 256
    wl = datagen.moe_nvfp4_workload(1004, DEV, T=T, H=H, I=I)
    t = wl.tensors
    ids, w = mxg.moe_route_noaux(t["logits"], t["bias"], 8, 4, TOPK, 2.5)
    mm, _ = mxg.moe_dispatch(ids, E, 1 << 20)
    cap = max(16, -(-int(mm.max().item()) // 16) * 16)
    assert (cap <= 32) == (T == 16)
    _check(wl, T, H, I, E, ids, w, cap, what)


def test_moe_nvfp4_interleaved_w13_tiled_kernel():
    """More than 1024 experts: GEMM1 with max_m > 32 runs on the tiled kernel."""
    E, T, H, I = 1032, 48, 256, 128
    wl = datagen.moe_nvfp4_workload(1005, DEV, T=T, H=H, I=I, E=E)
    # every token to experts 3, 100, 517, 518, 700, 1000, 1024, 1031: 48 rows each
    ids = torch.tensor([3, 100, 517, 518, 700, 1000, 1024, 1031], dtype=torch.int32,
                       device=DEV).repeat(T, 1).contiguous()
    g = torch.Generator(device=DEV).manual_seed(11)
    w = (torch.rand((T, TOPK), generator=g, device=DEV) + 0.1).float().contiguous()
    _check(wl, T, H, I, E, ids, w, 48, "tiled kernel")


@pytest.mark.parametrize("T,H,I", [(16, 512, 256), (512, 512, 256), (64, 7168, 2048)])
def test_moe_nvfp4_interleaved_w13_against_oracle(T, H, I):
    """The interleaved-W13 layer checked against the oracle directly: the GPU runs on the
    interleaved copy, the oracle on the logical (stacked) weights, stage by stage."""
    import oracle
    from _helpers import bf16_tensor_bits, np_
    from _moe_check import check_nvfp4_layer
    mxg = _mxg()
    E = 256
    log(f"interleaved W13 against the oracle: T={T} H={H} I={I}")
    wl = datagen.moe_nvfp4_workload(1004, DEV, T=T, H=H, I=I)
    t, s = wl.tensors, wl.scalars
    ids, w = mxg.moe_route_noaux(t["logits"], t["bias"], 8, 4, TOPK, 2.5)
    mm, _ = mxg.moe_dispatch(ids, E, 1 << 20)
    cap = max(16, -(-int(mm.max().item()) // 16) * 16)
    masked_m, row = mxg.moe_dispatch(ids, E, cap)
    w13_il = mxg.moe_interleave_w13(t["w13"])
    sf_il = mxg.moe_interleave_w13(t["w13_sf"])
    y = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    dbg_h = torch.full((E, cap, I), float("nan"), dtype=torch.float32, device=DEV)
    dbg_g1 = torch.full((E, cap, 2 * I), float("nan"), dtype=torch.float32, device=DEV)
    d = mxg.make_moe_desc(mxg.MXG_MOE_NVFP4, T, H, I, E, TOPK, cap, t["x"], w13_il, sf_il, t["w2"], t["w2_sf"],
                          ids, w, masked_m, row, y, g_x=s["g_x"], g_w13=t["g_w13"], g_w2=t["g_w2"],
                          g_h=s["g_h"], w13_layout=mxg.MXG_W13_INTERLEAVED16, dbg_h=dbg_h, dbg_g1=dbg_g1)
    off = mxg.moe_expert_forward_workspace_layout(d)
    ws = torch.empty((off[5],), dtype=torch.uint8, device=DEV)
    mxg.moe_expert_forward(d, ws)
    torch.cuda.synchronize()
    ids_h, row_h = np_(ids), np_(row)
    ids_o, w_o = oracle.route_noaux(np_(t["logits"]), np_(t["bias"]), 8, 4, TOPK, 2.5)
    assert np.array_equal(ids_h, ids_o)

    def region(i, shape):
        n = int(np.prod(shape))
        return lambda e: np_(ws[off[i] + e * n: off[i] + (e + 1) * n]).reshape(shape)
    ga, gs = region(0, (cap, H // 2)), region(1, (cap, H // 16))
    hc, hs = region(2, (cap, I // 2)), region(3, (cap, I // 16))
    check_nvfp4_layer(
        x=np_(t["x"].float()), g_x=s["g_x"], ids=ids_h, w=np_(w), row=row_h, max_m=cap, I=I,
        weights=lambda e: (np_(t["w13"][e]), np_(t["w13_sf"][e]), np_(t["w2"][e]), np_(t["w2_sf"][e])),
        g_w13=np_(t["g_w13"]), g_w2=np_(t["g_w2"]), g_h=s["g_h"],
        gathered=lambda e: (ga(e), gs(e), hc(e), hs(e)), h_pre=lambda e: np_(dbg_h[e]),
        y_bits=bf16_tensor_bits(y), toks=np.arange(T), what=f"interleaved W13 T={T} H={H}",
        g1=lambda e: np_(dbg_g1[e]))
