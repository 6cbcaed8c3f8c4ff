"""moe_expert_forward_noalloc (workspace in the library's own device scratch) against
moe_expert_forward with a caller workspace: y bit for bit, on two calls in a row, the
second with a smaller layer, for both precisions.  A layer larger than the scratch is
refused before any GPU work."""
import ctypes

import numpy as np
import pytest
import torch

import datagen
import fp8_grouped_gemm_nvfp4_amd as mxg
from _helpers import log

DEV = torch.device("cuda:0") if torch.cuda.is_available() else None
E, TOPK = 256, 8


def _layer_desc(precision, T, H, I, seed):
    if precision == "nvfp4":
        wl = datagen.moe_nvfp4_workload(seed, DEV, T=T, H=H, I=I)
    else:
        wl = datagen.moe_fp8_workload(seed, DEV, T=T, H=H, I=I)
    t, s = wl.tensors, wl.scalars
    ids, w = mxg.moe_route_noaux(t["logits"], t["bias"], 8, 4, TOPK, 2.5)
    mm, _ = mxg.moe_dispatch(ids, E, 1 << 20)
    cap = max(16, -(-int(mm.max().item()) // 16) * 16)
    masked_m, row = mxg.moe_dispatch(ids, E, cap)
    keep = [t, ids, w, masked_m, row]

    def desc(y):
        if precision == "nvfp4":
            return mxg.make_moe_desc(mxg.MXG_MOE_NVFP4, T, H, I, E, TOPK, cap, t["x"], t["w13"], t["w13_sf"],
                                     t["w2"], t["w2_sf"], ids, w, masked_m, row, y, g_x=s["g_x"],
                                     g_w13=t["g_w13"], g_w2=t["g_w2"], g_h=s["g_h"])
        return mxg.make_moe_desc(mxg.MXG_MOE_FP8_BLOCK128, T, H, I, E, TOPK, cap, t["xq"], t["w13"], t["w13_s"],
                                 t["w2"], t["w2_s"], ids, w, masked_m, row, y, x_scale=t["xs"])
    return desc, cap, keep


@pytest.mark.gpu
@pytest.mark.parametrize("precision", ["nvfp4", "fp8"])
def test_noalloc_matches_workspace_entry_point(precision):
    for T, H, I, seed in [(64, 7168, 2048, 1004), (16, 1024, 512, 4100)]:
        log(f"no-alloc MoE layer {precision} T={T} H={H} I={I}")
        desc, cap, keep = _layer_desc(precision, T, H, I, seed)
        y_ref = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
        y_na = torch.full((T, H), float("nan"), dtype=torch.bfloat16, device=DEV)
        d_ref, d_na = desc(y_ref), desc(y_na)
        need = mxg.moe_expert_forward_workspace_size(d_ref)
        assert need <= mxg.lib().moe_expert_forward_workspace_size(ctypes.byref(d_na))
        ws = torch.empty((need,), dtype=torch.uint8, device=DEV)
        mxg.moe_expert_forward(d_ref, ws)
        mxg.moe_expert_forward_noalloc(d_na)
        torch.cuda.synchronize()
        assert not torch.isnan(y_ref.float()).any()
        assert torch.equal(y_na.view(torch.int16), y_ref.view(torch.int16)), \
            f"{precision} T={T}: the no-alloc entry point differs from the workspace one"
        log(f"  max_m={cap}, workspace {need / 2**20:.1f} MiB: bit-identical")


def test_noalloc_rejects_oversized_layer():
    # full-size layer at capacity 64: far beyond the scratch; refused before any HIP call
    d = mxg.MoeDesc(mxg.MXG_MOE_NVFP4, 64, 7168, 2048, 256, 8, 64, 16, None, 0.01, 16, 16, 16, 16, 16, 16,
                    1024.0, 16, 16, 16, 16, 16, None, 0, None)
    assert mxg.lib().moe_expert_forward_workspace_size(ctypes.byref(d)) > 192 << 20
    assert mxg.lib().moe_expert_forward_noalloc(ctypes.byref(d), None) == mxg.MXG_ERR_WORKSPACE
    assert b"scratch" in mxg.lib().mxg_last_error()
