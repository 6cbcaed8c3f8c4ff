"""GPU parity of routing, dispatch and NVFP4 quantization: bit-exact against the oracle."""
import numpy as np
import pytest
import torch

import datagen
import oracle
from _helpers import log, np_

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0") if torch.cuda.is_available() else None


def _mxg():
    import fp8_grouped_gemm_nvfp4_amd as mxg
    return mxg


@pytest.mark.parametrize("T,ng,tg,k,seed", [
    (4096, 8, 4, 8, 3), (8192, 8, 4, 8, 4), (64, 8, 4, 8, 5), (1, 8, 4, 8, 6),
    (333, 1, 1, 8, 7), (200, 4, 2, 6, 8), (100, 2, 1, 1, 9),
])
def test_route_bit_exact(T, ng, tg, k, seed):
    log(f"route T={T} n_group={ng} topk_group={tg} top_k={k}")
    gen = datagen.generator(seed, DEV)
    logits, bias = datagen.router_inputs(gen, T, 256, DEV)
    if T >= 64:
        logits[: T // 8] = torch.round(logits[: T // 8] * 4) / 4  # planted ties
    ids, w = _mxg().moe_route_noaux(logits, bias, ng, tg, k, 2.5)
    torch.cuda.synchronize()
    ids_o, w_o = oracle.route_noaux(np_(logits), np_(bias), ng, tg, k, 2.5)
    ids_g, w_g = np_(ids), np_(w)
    bad = np.nonzero((ids_g != ids_o).any(axis=1))[0]
    assert len(bad) == 0, f"{len(bad)} tokens differ, first {bad[:3]}: {ids_g[bad[0]]} vs {ids_o[bad[0]]}"
    assert np.array_equal(w_g.view(np.uint32), w_o.view(np.uint32)), "weights differ"


@pytest.mark.parametrize("T,k,max_m", [(8, 8, 8), (64, 8, 64), (4096, 8, 256), (8192, 8, 512), (1000, 3, 5)])
def test_dispatch_bit_exact(T, k, max_m):
    log(f"dispatch T={T} top_k={k} max_m={max_m}")
    gen = datagen.generator(T + k, DEV)
    ids = datagen.distinct_topk_ids(gen, T, 256, k, DEV)
    mm, row, offs = _mxg().moe_dispatch(ids, 256, max_m, with_offsets=True)
    torch.cuda.synchronize()
    mm_o, row_o = oracle.dispatch(np_(ids), 256, max_m)
    assert np.array_equal(np_(mm), mm_o)
    assert np.array_equal(np_(row), row_o)
    # offsets: exclusive prefix sum of masked_m (closed form from the oracle's counts)
    assert np.array_equal(np_(offs), np.concatenate([[0], np.cumsum(mm_o)]))


@pytest.mark.parametrize("T,E,k,max_m,unaligned", [
    (128, 256, 8, 16, False),    # exactly one 1024-slot chunk
    (129, 16, 8, 40, True),      # one slot past the chunk, 16 experts, ids not 16-byte aligned
    (2048, 7, 3, 4096, True),    # few experts, six chunks, unaligned
    (300, 5000, 4, 3, False),    # more experts than the chunked kernel takes: one workgroup per expert
])
def test_dispatch_edges(T, E, k, max_m, unaligned):
    log(f"dispatch T={T} E={E} top_k={k} max_m={max_m}{' unaligned ids' if unaligned else ''}")
    gen = datagen.generator(4400 + T + E, DEV)
    ids = datagen.distinct_topk_ids(gen, T, E, k, DEV)
    if unaligned:  # the same ids 4 bytes past a 16-byte boundary
        buf = torch.empty((T * k + 1,), dtype=torch.int32, device=DEV)
        buf[1:] = ids.flatten()
        ids = buf[1:].view(T, k)
        assert ids.data_ptr() % 16 == 4
    mm, row = _mxg().moe_dispatch(ids, E, max_m)
    torch.cuda.synchronize()
    mm_o, row_o = oracle.dispatch(np_(ids), E, max_m)
    assert np.array_equal(np_(mm), mm_o)
    assert np.array_equal(np_(row), row_o)


def _quant_inputs(gen, rows, K):
    x = torch.randn((rows, K), generator=gen, device=DEV) * 3
    x[0] = 0.0
    x[1, ::2] = -0.0
    x[2] = 1e30
    x[3] = torch.randn((K,), generator=gen, device=DEV) * 1e-30
    x[4, ::16] = 6.0
    x[5] = torch.arange(K, device=DEV, dtype=torch.float32) / 8 - K / 16
    return x


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("g", [1.0, 0.0123, 37.5])
def test_quantize_bit_exact(dtype, g):
    log(f"NVFP4 quantize dtype={dtype} g={g}")
    gen = datagen.generator(17, DEV)
    x = _quant_inputs(gen, 512, 1024).to(dtype)
    codes, sf = _mxg().mx_quantize_nvfp4(x, g)
    torch.cuda.synchronize()
    c_o, s_o = oracle.quantize_nvfp4(np_(x.float()), g)
    assert np.array_equal(np_(sf), s_o)
    assert np.array_equal(np_(codes), c_o)


def test_quantize_all_bf16_values():
    """Every finite bf16 value, in blocks whose maxima sweep the scale range."""
    log("NVFP4 quantize over all finite bf16 values")
    bits = torch.arange(0, 0x10000, dtype=torch.int32, device=DEV)
    keep = (bits & 0x7F80) != 0x7F80
    v = bits[keep].to(torch.int16).view(torch.bfloat16)
    n = (v.numel() // 16) * 16
    x = v[:n].reshape(-1, 16)
    x = x[torch.randperm(x.shape[0], generator=datagen.generator(3, DEV), device=DEV)].contiguous()
    for g in (1.0, 2.0 ** -100, 1e-3):
        codes, sf = _mxg().mx_quantize_nvfp4(x, g)
        torch.cuda.synchronize()
        c_o, s_o = oracle.quantize_nvfp4(np_(x.float()), g)
        assert np.array_equal(np_(sf), s_o), g
        assert np.array_equal(np_(codes), c_o), g


@pytest.mark.parametrize("T,H,k,max_m", [(300, 7168, 8, 12), (77, 2048, 6, 5), (50, 1024, 4, 3), (40, 1024, 2, 2),
                                         (300, 512, 8, 12), (60, 1024, 3, 4)])
def test_quantize_gather_bit_exact(T, H, k, max_m):
    """Both launch shapes: one wave per 64 blocks of a token with top_k fixed at compile time
    (H % 1024 == 0, top_k in {2, 4, 6, 8}) and one thread per block otherwise."""
    log(f"quantize + gather into the masked layout, T={T} top{k} H={H} max_m={max_m} (some slots dropped)")
    gen = datagen.generator(19 + T + k, DEV)
    E = 256
    ids = datagen.distinct_topk_ids(gen, T, E, k, DEV)
    x = datagen.bf16_normal(gen, (T, H), DEV)
    g_x = datagen.global_scale_from_amax(x)
    mxg = _mxg()
    mm, row = mxg.moe_dispatch(ids, E, max_m)
    a = torch.full((E, max_m, H // 2), 0xEE, dtype=torch.uint8, device=DEV)
    a_sf = torch.full((E, max_m, H // 16), 0xEE, dtype=torch.uint8, device=DEV)
    mxg.moe_quantize_gather_nvfp4(x, g_x, ids, row, E, max_m, a=a, a_sf=a_sf)
    torch.cuda.synchronize()
    c_o, s_o = oracle.quantize_nvfp4(np_(x.float()), g_x)
    mm_o, row_o = oracle.dispatch(np_(ids), E, max_m)
    a_h, asf_h, ids_h = np_(a), np_(a_sf), np_(ids)
    filled = np.zeros((E, max_m), bool)
    for t in range(T):
        for j in range(k):
            e, r = ids_h[t, j], row_o[t, j]
            if r < max_m:
                assert np.array_equal(a_h[e, r], c_o[t]) and np.array_equal(asf_h[e, r], s_o[t])
                filled[e, r] = True
    assert (a_h[~filled] == 0xEE).all() and (asf_h[~filled] == 0xEE).all()
    assert filled.sum() == mm_o.sum()


@pytest.mark.parametrize("T,k,max_m,H", [(8, 8, 8, 7168), (1, 8, 4, 1024), (32, 8, 16, 512), (37, 4, 3, 256),
                                         (64, 8, 16, 512)])
def test_dispatch_quantize_gather_fused_matches_two_calls(T, k, max_m, H):
    """The one-launch small-batch path (T * k <= 256) and the two-kernel path it falls back
    to (T * k = 512) give masked_m, row and every dispatched row bit for bit as
    moe_dispatch + moe_quantize_gather_nvfp4."""
    import fp8_grouped_gemm_nvfp4_amd as mxg
    E = 256
    log(f"fused dispatch + quantize-gather: T={T} k={k} max_m={max_m} H={H}")
    gen = datagen.generator(77 + T, DEV)
    ids = datagen.distinct_topk_ids(gen, T, E, k, DEV)
    x = datagen.bf16_normal(gen, (T, H), DEV)
    g = datagen.global_scale_from_amax(x)
    mm0, row0 = mxg.moe_dispatch(ids, E, max_m)
    a0, sf0 = mxg.moe_quantize_gather_nvfp4(x, g, ids, row0, E, max_m)
    mm1, row1, a1, sf1 = mxg.moe_dispatch_quantize_gather_nvfp4(x, g, ids, E, max_m)
    torch.cuda.synchronize()
    assert torch.equal(mm0, mm1) and torch.equal(row0, row1)
    mm = mm0.cpu().numpy()
    a0, a1, sf0, sf1 = a0.cpu().numpy(), a1.cpu().numpy(), sf0.cpu().numpy(), sf1.cpu().numpy()
    for e in np.nonzero(mm)[0]:
        m = int(mm[e])
        assert np.array_equal(a0[e, :m], a1[e, :m]) and np.array_equal(sf0[e, :m], sf1[e, :m]), f"expert {e}"
    # and the one-launch path against the oracle itself
    ids_h = np_(ids)
    mm_o, row_o = oracle.dispatch(ids_h, E, max_m)
    assert np.array_equal(np_(mm1), mm_o) and np.array_equal(np_(row1), row_o)
    c_o, s_o = oracle.quantize_nvfp4(np_(x.float()), g)
    for t in range(T):
        for j in range(k):
            e, r = ids_h[t, j], row_o[t, j]
            if r < max_m:
                assert np.array_equal(a1[e, r], c_o[t]) and np.array_equal(sf1[e, r], s_o[t]), (t, j)
