"""Seeded synthetic inputs shared by the GPU path's tests/benchmark and the oracle.

This module holds only random draws and input preparation; none of the method's
arithmetic (no GEMM, no NVFP4 quantizer, no routing).  Tensors are produced with
torch generators on the requested device, so the large weight sets of the MoE
workloads are drawn directly in HBM; the oracle always receives the very same bytes
(copied to the host), never a regenerated copy.

Distributions (the workloads' recipes):
  * NVFP4 operands: e2m1 codes i.i.d. uniform over all 16 codes (so each packed byte
    is uniform over 0..255), e4m3 block scales 2^u with u i.i.d. uniform in [-4, 4]
    (e4m3 byte (u + 7) << 3), fixed fp32 global scales.
  * activations: bf16 N(0, 1); router logits fp32 N(0, 1); router bias fp32 N(0, 0.01)
    (second parameter = standard deviation); FP8 weights from N(0, 0.02).
  * FP8 input preparation (not part of the timed path): per 1x128 row block or per
    128x128 weight block, scale = amax / 448 (1 if amax == 0) and codes = the
    float8_e4m3fn cast of value / scale (torch's cast, round to nearest even).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

E4M3_MAX = 448.0


def generator(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def uniform_bytes(gen, shape, device):
    return torch.randint(0, 256, tuple(shape), generator=gen, device=device, dtype=torch.int32).to(torch.uint8)


def pow2_scales(gen, shape, device, lo=-4, hi=4):
    """e4m3 bytes of 2^u, u uniform integer in [lo, hi]."""
    u = torch.randint(lo, hi + 1, tuple(shape), generator=gen, device=device, dtype=torch.int32)
    return ((u + 7) << 3).to(torch.uint8)


def nvfp4_uniform(gen, rows_shape, K, device):
    """Codes [*rows, K/2] uniform over all bytes; scales [*rows, K/16] = 2^U{-4..4}."""
    codes = uniform_bytes(gen, (*rows_shape, K // 2), device)
    sf = pow2_scales(gen, (*rows_shape, K // 16), device)
    return codes, sf


def bf16_normal(gen, shape, device, std=1.0):
    x = torch.randn(tuple(shape), generator=gen, device=device, dtype=torch.float32)
    if std != 1.0:
        x = x * std
    return x.to(torch.bfloat16)


def f32_normal(gen, shape, device, std=1.0):
    x = torch.randn(tuple(shape), generator=gen, device=device, dtype=torch.float32)
    return x * std if std != 1.0 else x


def distinct_topk_ids(gen, T, E, k, device):
    """k distinct experts per token, uniform: the first k of a random permutation
    (argsort of i.i.d. uniform keys)."""
    keys = torch.rand((T, E), generator=gen, device=device)
    return torch.argsort(keys, dim=1)[:, :k].to(torch.int32).contiguous()


def global_scale_from_amax(x: torch.Tensor) -> float:
    """fp32 global dequantization scale amax(|x|) / (6 * 448), the usual NVFP4 choice."""
    amax = x.float().abs().max().to(torch.float32)
    return float((amax / torch.tensor(6.0 * E4M3_MAX, dtype=torch.float32, device=amax.device)).item())


def fp8_rowblock_quant(x_bf16: torch.Tensor):
    """Per 1x128 block of each row: fp32 scale = amax / 448 and e4m3 codes."""
    T, H = x_bf16.shape
    xb = x_bf16.float().view(T, H // 128, 128)
    amax = xb.abs().amax(dim=2)
    scale = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
    q = (xb / scale[..., None]).to(torch.float8_e4m3fn).view(torch.uint8).view(T, H)
    return q.contiguous(), scale.contiguous()


def fp8_weight_normal(gen, E, N, K, device, std=0.02, chunk=8):
    """FP8 weights [E, N, K] from N(0, std) with fp32 scales [E, N/128, K/128]."""
    q = torch.empty((E, N, K), dtype=torch.uint8, device=device)
    s = torch.empty((E, N // 128, K // 128), dtype=torch.float32, device=device)
    for e0 in range(0, E, chunk):
        e1 = min(E, e0 + chunk)
        w = torch.randn((e1 - e0, N, K), generator=gen, device=device, dtype=torch.float32) * std
        wb = w.view(e1 - e0, N // 128, 128, K // 128, 128)
        amax = wb.abs().amax(dim=(2, 4))
        sc = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
        qb = (wb / sc[:, :, None, :, None]).to(torch.float8_e4m3fn).view(torch.uint8)
        q[e0:e1] = qb.view(e1 - e0, N, K)
        s[e0:e1] = sc
        del w, wb, qb
    return q, s


# --------------------------------------------------------------------------- workloads
@dataclass
class Workload:
    name: str
    tensors: dict = field(default_factory=dict)
    scalars: dict = field(default_factory=dict)


def masked_gemm_workload(seed, device, G=4, max_m=64, N=512, K=1024, g_a=0.5, g_b=0.25,
                         masked_m=None):
    """NVFP4 masked grouped NT GEMM: per-group masked_m uniform in [0, max_m]."""
    gen = generator(seed, device)
    a, a_sf = nvfp4_uniform(gen, (G, max_m), K, device)
    b, b_sf = nvfp4_uniform(gen, (G, N), K, device)
    if masked_m is None:
        mm = torch.randint(0, max_m + 1, (G,), generator=gen, device=device, dtype=torch.int32)
    else:
        mm = torch.as_tensor(masked_m, dtype=torch.int32, device=device)
    alpha = torch.full((G,), g_a * g_b, dtype=torch.float32, device=device)
    return Workload(f"masked_nvfp4_g{G}_m{max_m}_n{N}_k{K}",
                    dict(a=a, a_sf=a_sf, b=b, b_sf=b_sf, masked_m=mm, alpha=alpha),
                    dict(G=G, max_m=max_m, N=N, K=K, g_a=g_a, g_b=g_b))


def hetero_gemm_workload(seed, device, shapes=((128, 4096, 7168), (1000, 2048, 7168),
                                               (4096, 7168, 2048), (37, 4096, 4096)),
                         g_a=0.5, g_b=0.25):
    """Heterogeneous NVFP4 grouped NT GEMM: one (M, N, K) per group."""
    gen = generator(seed, device)
    groups = []
    for (M, N, K) in shapes:
        a, a_sf = nvfp4_uniform(gen, (M,), K, device)
        b, b_sf = nvfp4_uniform(gen, (N,), K, device)
        groups.append(dict(M=M, N=N, K=K, a=a, a_sf=a_sf, b=b, b_sf=b_sf, alpha=g_a * g_b))
    name = "hetero_nvfp4_" + "_".join(f"{m}x{n}x{k}" for m, n, k in shapes)
    return Workload(name, dict(groups=groups), dict(g_a=g_a, g_b=g_b))


def decode_gemm1_workload(seed, device, E=256, T=8, top_k=8, H=7168, I=2048, g_w=0.25):
    """Decode-shaped MoE GEMM1: T tokens routed top-k to E experts (ids from the seed),
    bf16 activations quantized on the fly, W13 [E, 2I, H] NVFP4 with gate and up stacked."""
    gen = generator(seed, device)
    ids = distinct_topk_ids(gen, T, E, top_k, device)
    x = bf16_normal(gen, (T, H), device)
    w13, w13_sf = nvfp4_uniform(gen, (E, 2 * I), H, device)
    g_x = global_scale_from_amax(x)
    return Workload(f"decode_gemm1_nvfp4_e{E}_t{T}_top{top_k}_h{H}_n{2 * I}",
                    dict(ids=ids, x=x, w13=w13, w13_sf=w13_sf),
                    dict(E=E, T=T, top_k=top_k, H=H, N=2 * I, g_x=g_x, g_w=g_w))


def gemv_w4a16_workload(seed, device, M=1, N=4096, K=4096, g_w=0.25):
    """Decode GEMV with NVFP4 weights and bf16 activations (the nvfp4_gemv W4A16 case):
    x [M, K] bf16 ~ N(0, 1), W codes [N, K/2] uniform bytes, scales 2^U{-4..4}."""
    gen = generator(seed, device)
    x = bf16_normal(gen, (M, K), device)
    w, w_sf = nvfp4_uniform(gen, (N,), K, device)
    return Workload(f"gemv_w4a16_m{M}_n{N}_k{K}", dict(x=x, w=w, w_sf=w_sf), dict(M=M, N=N, K=K, g_w=g_w))


def router_inputs(gen, T, E, device):
    logits = f32_normal(gen, (T, E), device)
    bias = f32_normal(gen, (E,), device, std=0.01)
    return logits, bias


def moe_fp8_workload(seed, device, T=4096, H=7168, I=2048, E=256, top_k=8):
    """DeepSeek-V3-style FP8 MoE layer: fp8 activations (1x128 scales), W13 [E, 2I, H]
    and W2 [E, H, I] fp8 with 128x128 scales, router logits and bias."""
    gen = generator(seed, device)
    logits, bias = router_inputs(gen, T, E, device)
    x = bf16_normal(gen, (T, H), device)
    xq, xs = fp8_rowblock_quant(x)
    del x
    w13, w13_s = fp8_weight_normal(gen, E, 2 * I, H, device)
    w2, w2_s = fp8_weight_normal(gen, E, H, I, device)
    return Workload(f"moe_fp8_t{T}_h{H}_i{I}_e{E}_top{top_k}",
                    dict(logits=logits, bias=bias, xq=xq, xs=xs, w13=w13, w13_s=w13_s, w2=w2, w2_s=w2_s),
                    dict(T=T, H=H, I=I, E=E, top_k=top_k, n_group=8, topk_group=4, rsf=2.5))


def moe_nvfp4_workload(seed, device, T=64, H=7168, I=2048, E=256, top_k=8, g_w=0.25, g_h=1024.0):
    """NVFP4 MoE layer: bf16 activations quantized in the layer, NVFP4 W13/W2 with
    per-expert fp32 global scales, a fixed global scale g_h for the intermediate."""
    gen = generator(seed, device)
    logits, bias = router_inputs(gen, T, E, device)
    x = bf16_normal(gen, (T, H), device)
    w13, w13_sf = nvfp4_uniform(gen, (E, 2 * I), H, device)
    w2, w2_sf = nvfp4_uniform(gen, (E, H), I, device)
    g_w13 = torch.full((E,), g_w, dtype=torch.float32, device=device)
    g_w2 = torch.full((E,), g_w, dtype=torch.float32, device=device)
    g_x = global_scale_from_amax(x)
    return Workload(f"moe_nvfp4_t{T}_h{H}_i{I}_e{E}_top{top_k}",
                    dict(logits=logits, bias=bias, x=x, w13=w13, w13_sf=w13_sf, w2=w2, w2_sf=w2_sf,
                         g_w13=g_w13, g_w2=g_w2),
                    dict(T=T, H=H, I=I, E=E, top_k=top_k, n_group=8, topk_group=4, rsf=2.5,
                         g_x=g_x, g_h=g_h))
