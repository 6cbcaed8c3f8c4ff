"""GPU parity of the NVFP4-weight x bf16-activation GEMV (W4A16) against the oracle:
every output at Llama-3-sized shapes, sampled columns of an LM-head-sized one, N tails,
the largest activation block, activation rows at the edges of the fp16 scaling, and
the bytes past the output left untouched."""
import numpy as np
import pytest
import torch

import datagen
import oracle
from _helpers import (SENT_BF16, SENT_F32, assert_within, bf16_from_bits_np, bf16_tensor_bits, log, np_,
                      sentinel_bf16, sentinel_f32, ulp_f32)

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0") if torch.cuda.is_available() else None


def _mxg():
    import fp8_grouped_gemm_nvfp4_amd as mxg
    return mxg


def _run(x, w, w_sf, g_w, N, out_dtype, pad=64):
    M = x.shape[0]
    buf = (sentinel_bf16 if out_dtype == torch.bfloat16 else sentinel_f32)((M * N + pad,), DEV)
    out = buf[: M * N].view(M, N)
    _mxg().mx_gemv_nvfp4_w4a16(x, w, w_sf, g_w, out=out)
    torch.cuda.synchronize()
    if out_dtype == torch.bfloat16:
        tail = bf16_tensor_bits(buf[M * N:])
        assert (tail == SENT_BF16).all(), "bytes past the output were written"
        return bf16_from_bits_np(bf16_tensor_bits(out))
    tail = np_(buf[M * N:]).view(np.uint32)
    assert (tail == (SENT_F32 & 0xFFFFFFFF)).all(), "bytes past the output were written"
    return np_(out).astype(np.float64)


def _check(x, w, w_sf, g_w, got, cols, what, out_dtype):
    x_bits = bf16_tensor_bits(x)
    y, s = oracle.gemv_nvfp4_w4a16(x_bits, np_(w[cols]), np_(w_sf[cols]), g_w)
    ulp = None if out_dtype == torch.bfloat16 else ulp_f32
    kw = {} if ulp is None else dict(ulp=ulp)
    assert_within(got[:, cols], y, s, what, **kw)


@pytest.mark.parametrize("M,N,K,out_dtype", [
    (1, 4096, 4096, torch.bfloat16),     # q / o projection
    (1, 14336, 4096, torch.bfloat16),    # gate / up projection
    (1, 4096, 14336, torch.bfloat16),    # down projection
    (4, 520, 8192, torch.bfloat16),      # largest activation block, N tail inside a 16-column unit
    (3, 37, 1024, torch.float32),        # 3 units, one chunk per wave
    (2, 100, 2048, torch.float32),       # N % 16 == 4
])
def test_gemv_w4a16_shapes(M, N, K, out_dtype):
    log(f"W4A16 GEMV M={M} N={N} K={K} {out_dtype}")
    wl = datagen.gemv_w4a16_workload(4000 + N + K + M, DEV, M=M, N=N, K=K)
    t, g_w = wl.tensors, wl.scalars["g_w"]
    got = _run(t["x"], t["w"], t["w_sf"], g_w, N, out_dtype)
    _check(t["x"], t["w"], t["w_sf"], g_w, got, np.arange(N), f"gemv M={M} N={N} K={K}", out_dtype)


def test_gemv_w4a16_lm_head_sampled():
    M, N, K = 1, 128256, 4096
    log(f"W4A16 GEMV LM-head size M={M} N={N} K={K}, 2048 sampled columns")
    wl = datagen.gemv_w4a16_workload(4100, DEV, M=M, N=N, K=K)
    t, g_w = wl.tensors, wl.scalars["g_w"]
    got = _run(t["x"], t["w"], t["w_sf"], g_w, N, torch.bfloat16)
    cols = np.unique(np.concatenate([np.random.default_rng(5).choice(N, 2000, replace=False),
                                     np.arange(N - 48, N)]))
    _check(t["x"], t["w"], t["w_sf"], g_w, got, cols, "gemv lm head", torch.bfloat16)


def test_gemv_w4a16_activation_edges_and_general_scales():
    # row 0 all zero; row 1 bf16 subnormals only; row 2 magnitudes near 2^100; row 3 mixed
    # magnitudes spanning 2^-40 .. 2^8 (elements far below the row maximum); general
    # (non power of two, signed) e4m3 weight scales
    M, N, K = 4, 272, 4096
    log(f"W4A16 GEMV activation edge rows and general scales M={M} N={N} K={K}")
    g = datagen.generator(4200, DEV)
    x = torch.zeros((M, K), dtype=torch.float32, device=DEV)
    x[2] = torch.randn(K, generator=g, device=DEV) * 2.0 ** 100
    e = torch.randint(-40, 9, (K,), generator=g, device=DEV).float()
    x[3] = torch.randn(K, generator=g, device=DEV) * torch.pow(2.0, e)
    x = x.to(torch.bfloat16)
    # subnormal bf16 bit patterns (exponent field 0), built as integers
    sub = torch.randint(1, 128, (K,), generator=g, device=DEV, dtype=torch.int32)
    sub = sub | (torch.randint(0, 2, (K,), generator=g, device=DEV, dtype=torch.int32) << 15)
    x[1] = sub.to(torch.int16).view(torch.bfloat16)
    w = datagen.uniform_bytes(g, (N, K // 2), DEV)
    w_sf = torch.randint(0x18, 0x58, (N, K // 16), generator=g, device=DEV, dtype=torch.int32)
    w_sf = (w_sf | (torch.randint(0, 2, (N, K // 16), generator=g, device=DEV, dtype=torch.int32) << 7)).to(torch.uint8)
    bits = bf16_tensor_bits(x)
    assert ((bits[1] & 0x7F80) == 0).all() and (bits[1] != 0).any(), "row 1 holds subnormals"
    for out_dtype in (torch.float32, torch.bfloat16):
        got = _run(x, w, w_sf, 0.375, N, out_dtype)
        _check(x, w, w_sf, 0.375, got, np.arange(N), f"gemv edges {out_dtype}", out_dtype)
        assert (got[0] == 0).all()


def test_gemv_w4a16_repeatable_and_cu_limit():
    M, N, K = 2, 2048, 4096
    wl = datagen.gemv_w4a16_workload(4300, DEV, M=M, N=N, K=K)
    t, g_w = wl.tensors, wl.scalars["g_w"]
    outs = []
    for cu in (0, 0, 7):
        out = torch.empty((M, N), dtype=torch.float32, device=DEV)
        _mxg().mx_gemv_nvfp4_w4a16(t["x"], t["w"], t["w_sf"], g_w, out=out, cu_limit=cu)
        torch.cuda.synchronize()
        outs.append(np_(out))
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))
    assert np.array_equal(outs[0].view(np.uint32), outs[2].view(np.uint32)), "result depends on the grid"
