"""Shared test helpers: the parity tolerance and tensor <-> numpy plumbing.

Tolerance for a floating-point output element against the oracle's unrounded fp64
value y* (S = sum_k |a_k * b_k| over fully decoded operands, including alpha):
    |y_gpu - y*| <= 1e-5 * S + ulp(|y*|)
with ulp the bf16 (8-bit significand) or fp32 (24-bit) unit in the last place at |y*|.
"""
import sys

import numpy as np
import torch

SENT_BF16 = 0x7FC1
SENT_F32 = 0x7FC00001


def ulp_bf16(v):
    a = np.abs(np.asarray(v, np.float64))
    return np.where(a < 2.0 ** -126, 2.0 ** -133, 2.0 ** (np.floor(np.log2(np.maximum(a, 2.0 ** -126))) - 7))


def ulp_f32(v):
    a = np.abs(np.asarray(v, np.float64))
    return np.where(a < 2.0 ** -126, 2.0 ** -149, 2.0 ** (np.floor(np.log2(np.maximum(a, 2.0 ** -126))) - 23))


def within(gpu_vals, ystar, S, ulp=ulp_bf16, rel=1e-5, extra=0.0):
    """Boolean mask of elements inside the tolerance (plus an `extra` allowance)."""
    g = np.asarray(gpu_vals, np.float64)
    return np.abs(g - ystar) <= rel * S + ulp(ystar) + extra


def assert_within(gpu_vals, ystar, S, what, ulp=ulp_bf16, rel=1e-5, extra=0.0):
    ok = within(gpu_vals, ystar, S, ulp, rel, extra)
    if not ok.all():
        g = np.asarray(gpu_vals, np.float64)
        bad = np.argwhere(~ok)
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} of {ok.size} outside tolerance; first {i}: "
                             f"gpu={g[i]!r} oracle={ystar[i]!r} S={S[i]!r}")


def bf16_tensor_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_from_bits_np(bits) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def sentinel_bf16(shape, device):
    return torch.full(shape, SENT_BF16, dtype=torch.int32, device=device).to(torch.int16).view(torch.bfloat16)


def sentinel_f32(shape, device):
    return torch.full(shape, SENT_F32, dtype=torch.int64, device=device).to(torch.int32).view(torch.float32)


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def np_(t):
    return t.detach().cpu().numpy()
