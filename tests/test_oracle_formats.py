"""Pins for the oracle's format tables and encoders (CPU only).

The pages name e2m1 / e4m3fn / bf16 but do not define them; the pins use the
standard bit-field definitions, torch's own float8_e4m3fn / bfloat16 casts (library
routines) and brute force.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_e2m1_table_closed_form():
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    t = oracle.e2m1_table()
    assert list(t[:8]) == mags
    for c in range(8):
        assert t[c + 8] == -mags[c]
        assert np.signbit(t[c + 8])  # code 8 is -0
    assert all(t[c] < t[c + 1] for c in range(7))


def test_e4m3_table_matches_torch_decode():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    t = oracle.e4m3_table()
    nan = np.isnan(ref)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    assert np.array_equal(np.isnan(t), nan)
    assert np.array_equal(t[~nan], ref[~nan])
    assert np.array_equal(np.signbit(t[~nan]), np.signbit(ref[~nan]))


def test_golden_format_values():
    with open(os.path.join(GOLDEN, "formats.json")) as f:
        g = json.load(f)
    for code, val in g["e4m3"].items():
        assert oracle.e4m3_value(int(code, 16)) == float(Fraction(val))
    for code, val in g["e2m1"].items():
        assert oracle.e2m1_value(int(code, 16)) == float(Fraction(val))


def _nearest_e2m1_bruteforce(v):
    """Independent rule: walk the midpoints between consecutive magnitudes."""
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    a = abs(v)
    c = 0
    for i in range(7):
        mid = (mags[i] + mags[i + 1]) / 2
        if a > mid or (a == mid and (i + 1) % 2 == 0):
            c = i + 1
    return c | (8 if np.signbit(v) else 0)


def test_encode_e2m1_ties_and_saturation():
    cases = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6, 6.0: 7, 100.0: 7,
             0.2499: 0, 0.2501: 1, 0.7499: 1, 4.99: 6, 5.01: 7}
    for v, c in cases.items():
        assert oracle.encode_e2m1(v) == c, v
        assert oracle.encode_e2m1(-v) == c | 8, v
    assert oracle.encode_e2m1(np.inf) == 7 and oracle.encode_e2m1(-np.inf) == 15
    assert oracle.encode_e4m3_sat(np.array([np.inf, -np.inf])).tolist() == [0x7E, 0xFE]
    assert oracle.encode_e2m1(-0.0) == 8
    assert oracle.encode_e2m1(0.0) == 0


def test_encode_e2m1_bruteforce_dense():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.uniform(-8, 8, 20000), np.arange(-7, 7.01, 0.125),
                        np.arange(-7, 7.01, 0.25) + 1e-9])
    got = oracle.encode_e2m1(v)
    want = np.array([_nearest_e2m1_bruteforce(x) for x in v], np.uint8)
    assert np.array_equal(got, want)


def test_encode_e4m3_matches_torch_cast():
    # torch's fp32 -> float8_e4m3fn cast rounds to nearest even; it returns NaN rather
    # than saturating beyond 464, so compare on |v| <= 448 plus explicit saturation.
    rng = np.random.default_rng(1)
    mags = np.concatenate([
        np.exp(rng.uniform(np.log(1e-4), np.log(448), 50000)),
        np.arange(0, 1e-2, 2.0 ** -12),          # subnormal range incl. all midpoints
        oracle.e4m3_table()[:0x7F],                # exact codes
    ]).astype(np.float32)
    v = np.concatenate([mags, -mags]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle.encode_e4m3_sat(v.astype(np.float64))
    assert np.array_equal(got, ref)
    assert oracle.encode_e4m3_sat(np.array([449.0, 464.0, 1e9, -1e9])).tolist() == [0x7E, 0x7E, 0x7E, 0xFE]


def test_bf16_matches_torch_on_fp32_inputs():
    rng = np.random.default_rng(2)
    bits = rng.integers(0, 2 ** 32, 200000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    # add exact ties
    ties = (np.arange(1, 5000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    f = np.concatenate([f, ties, -ties])
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.bf16_bits(f.astype(np.float64))
    fin = np.isfinite(f)
    assert np.array_equal(got[fin], ref[fin])


def test_bf16_single_rounding_from_fp64():
    # 1 + 2^-8 + 2^-40 lies above the bf16 midpoint 1 + 2^-8; a detour through fp32
    # would land on the midpoint and tie to 1.0.  Direct rounding gives 1 + 2^-7.
    v = 1.0 + 2.0 ** -8 + 2.0 ** -40
    assert oracle.bf16_value(oracle.bf16_bits(np.array([v])))[0] == 1.0 + 2.0 ** -7
    assert oracle.bf16_bits(np.array([1.0 + 2.0 ** -8]))[0] == 0x3F80       # tie -> even
    assert oracle.bf16_bits(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 0x3F82   # tie -> even (up)
    assert oracle.bf16_bits(np.array([3.5e38]))[0] == 0x7F80                  # overflow
    assert oracle.bf16_bits(np.array([-0.0]))[0] == 0x8000
    assert oracle.bf16_bits(np.array([2.0 ** -133]))[0] == 0x0001             # smallest subnormal
    assert oracle.bf16_bits(np.array([2.0 ** -134]))[0] == 0x0000             # tie -> even (0)
