"""Captured-graph replay of the decode paths.

The grouped benchmarks of the Helion "pretuned_kernels" README replay pre-captured
graphs, with device pointer tables set up before capture.  Every library call is
stream-ordered and allocates nothing, so a whole step (dispatch, quantize-gather and the
masked GEMM; or routing, dispatch and the NVFP4 expert layer) can be captured once and
replayed.  Each replay must reproduce the eager result bit for bit: between replays the
outputs are overwritten with a sentinel by eager work and the stream is synchronized.
"""
import numpy as np
import pytest
import torch

import datagen
from _helpers import log

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0") if torch.cuda.is_available() else None
E, TOPK = 256, 8
REPLAYS = 3


def _mxg():
    import fp8_grouped_gemm_nvfp4_amd as mxg
    return mxg


def _capture(step):
    """Capture step() on a side stream after one eager warm-up call there."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    return g


def _bits(t):
    return t.view(torch.int16 if t.element_size() == 2 else torch.int32).clone()


def _replay_and_check(g, outs, refs, what):
    for r in range(REPLAYS):
        for o in outs:
            o.view(torch.uint8).fill_(0x7F)  # eager sentinel between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, ref, name in zip(outs, refs, what):
            assert torch.equal(_bits(o), ref), f"replay {r}: {name} differs from the eager result"


def test_graph_decode_gemm1_step():
    mxg = _mxg()
    log("graph replay: decode GEMM1 step, E=256 T=8 top-8 K=1024 N=512")
    wl = datagen.decode_gemm1_workload(1001, DEV, H=1024, I=256)
    t, s = wl.tensors, wl.scalars
    T, H, N, max_m = s["T"], s["H"], s["N"], 8
    alpha = torch.full((E,), np.float32(s["g_x"]) * np.float32(s["g_w"]), dtype=torch.float32, device=DEV)
    masked_m = torch.empty((E,), dtype=torch.int32, device=DEV)
    row = torch.empty((T, TOPK), dtype=torch.int32, device=DEV)
    a = torch.empty((E, max_m, H // 2), dtype=torch.uint8, device=DEV)
    a_sf = torch.empty((E, max_m, H // 16), dtype=torch.uint8, device=DEV)
    out = torch.zeros((E, max_m, N), dtype=torch.bfloat16, device=DEV)

    def step():
        mxg.moe_dispatch(t["ids"], E, max_m, masked_m=masked_m, row=row)
        mxg.moe_quantize_gather_nvfp4(t["x"], s["g_x"], t["ids"], row, E, max_m, a=a, a_sf=a_sf)
        mxg.mx_grouped_gemm_masked(a, a_sf, t["w13"], t["w13_sf"], alpha, masked_m, out)

    step()
    torch.cuda.synchronize()
    assert int(masked_m.sum().item()) == T * TOPK
    ref_mm, ref_row = _bits(masked_m), _bits(row)
    ref_a, ref_sf, ref_out = a.cpu().numpy(), a_sf.cpu().numpy(), _bits(out).cpu().numpy()
    g = _capture(step)
    mm = ref_mm.cpu().numpy()
    for r in range(REPLAYS):
        for o in (masked_m, row, a, a_sf, out):
            o.view(torch.uint8).fill_(0x7F)  # eager sentinel between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(masked_m), ref_mm) and torch.equal(_bits(row), ref_row), f"replay {r}: dispatch"
        got_a, got_sf, got = a.cpu().numpy(), a_sf.cpu().numpy(), _bits(out).cpu().numpy()
        for e in np.nonzero(mm)[0]:
            m = int(mm[e])
            assert np.array_equal(got_a[e, :m], ref_a[e, :m]), f"replay {r}: expert {e} codes"
            assert np.array_equal(got_sf[e, :m], ref_sf[e, :m]), f"replay {r}: expert {e} scales"
            assert np.array_equal(got[e, :m], ref_out[e, :m]), f"replay {r}: expert {e} output rows"
            assert (got[e, m:] == 0x7F7F).all(), f"replay {r}: expert {e} rows past masked_m written"


def test_graph_moe_nvfp4_decode_layer():
    mxg = _mxg()
    T, H, I = 16, 1024, 256
    log(f"graph replay: NVFP4 MoE layer T={T} H={H} I={I}")
    wl = datagen.moe_nvfp4_workload(1004, DEV, T=T, H=H, I=I)
    t, sc = wl.tensors, wl.scalars
    ids = torch.empty((T, TOPK), dtype=torch.int32, device=DEV)
    w = torch.empty((T, TOPK), dtype=torch.float32, device=DEV)
    cap = 16
    masked_m = torch.empty((E,), dtype=torch.int32, device=DEV)
    row = torch.empty((T, TOPK), dtype=torch.int32, device=DEV)
    y = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    d = mxg.make_moe_desc(mxg.MXG_MOE_NVFP4, T, H, I, E, TOPK, cap, t["x"], t["w13"], t["w13_sf"],
                          t["w2"], t["w2_sf"], ids, w, masked_m, row, y, g_x=sc["g_x"], g_w13=t["g_w13"],
                          g_w2=t["g_w2"], g_h=sc["g_h"])
    ws = torch.empty((mxg.moe_expert_forward_workspace_size(d),), dtype=torch.uint8, device=DEV)

    def step():
        mxg.moe_route_noaux(t["logits"], t["bias"], 8, 4, TOPK, 2.5, ids=ids, w=w)
        mxg.moe_dispatch(ids, E, cap, masked_m=masked_m, row=row)
        mxg.moe_expert_forward(d, ws)

    step()
    torch.cuda.synchronize()
    assert int(masked_m.max().item()) <= cap
    outs = [ids, w, masked_m, row, y]
    refs = [_bits(o) for o in outs]
    g = _capture(step)
    _replay_and_check(g, outs, refs, ["ids", "w", "masked_m", "row", "y"])
