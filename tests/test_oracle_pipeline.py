"""Pins for the oracle's weighted combine and its whole MoE-layer chains (CPU only).

The combine is checked against exact rational sums.  The layer chains are checked on
the case where the mixture-of-experts layer reduces to a dense MLP: one expert, top-1,
one group.  Routing then picks expert 0 with weight 2.5 * s / s = 2.5 for every token, and
y = bf16(2.5 * W2 . q(silu(Wg . x) * (Wu . x))).  The test computes that with numpy
float64 matmuls over operands it decodes itself and scipy's logistic function; q is
the quantizer, which has pins of its own in test_oracle_quant_route.py.  Further
checks: token separability (a permutation of the tokens permutes y) and capacity drops
(a dropped slot's term leaves the combine).
"""
from fractions import Fraction

import numpy as np
import pytest
import torch
from scipy.special import expit

import oracle

E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _e4m3_torch(codes):
    """e4m3fn decode by torch's float8_e4m3fn view (a library routine)."""
    c = torch.from_numpy(np.ascontiguousarray(codes, np.uint8))
    return c.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _dec_nvfp4(codes, sf):
    """Independent NVFP4 decode: closed-form e2m1 magnitudes, torch's e4m3fn for scales."""
    codes = np.asarray(codes, np.uint8)
    nib = np.stack([codes & 15, codes >> 4], axis=-1).reshape(*codes.shape[:-1], codes.shape[-1] * 2)
    mag = np.array(E2M1)[nib & 7]
    val = np.where(nib & 8, -mag, mag)
    return val * np.repeat(_e4m3_torch(sf), 16, axis=-1)


# ----------------------------------------------------------------------------- combine
def test_combine_bruteforce_fraction():
    rng = np.random.default_rng(50)
    n, k, H = 5, 8, 7
    o = rng.standard_normal((n, k, H)) * np.exp2(rng.integers(-30, 30, (n, k, H)))
    so = np.abs(o) * rng.uniform(1, 3, (n, k, H))
    w = rng.uniform(-1, 3, (n, k)).astype(np.float32)
    kept = rng.random((n, k)) < 0.8
    kept[0] = True
    kept[1] = False
    ystar, S = oracle._combine_tokens(o, so, w, kept)
    for p in range(n):
        for h in range(H):
            terms = [Fraction(float(w[p, j])) * Fraction(o[p, j, h]) for j in range(k) if kept[p, j]]
            exact = sum(terms, Fraction(0))
            mag = sum((abs(t) for t in terms), Fraction(0))
            # k sequential fp64 additions of exactly representable-or-rounded products
            assert abs(Fraction(ystar[p, h]) - exact) <= Fraction(2 * k) * Fraction(2) ** -53 * mag
            sx = sum((abs(Fraction(float(w[p, j]))) * Fraction(so[p, j, h]) for j in range(k) if kept[p, j]),
                     Fraction(0))
            assert abs(Fraction(S[p, h]) - sx) <= Fraction(2 * k) * Fraction(2) ** -53 * sx
    assert np.all(ystar[1] == 0) and np.all(S[1] == 0)      # every slot dropped: y = 0


def test_combine_exact_on_dyadic_inputs():
    # bf16-weight-like dyadic values: every product and partial sum is exact in fp64
    rng = np.random.default_rng(51)
    n, k, H = 4, 8, 16
    o = rng.integers(-2 ** 20, 2 ** 20, (n, k, H)) * 2.0 ** -12
    w = (rng.integers(-2 ** 10, 2 ** 10, (n, k)) * 2.0 ** -9).astype(np.float32)
    kept = np.ones((n, k), bool)
    ystar, _ = oracle._combine_tokens(o, np.abs(o), w, kept)
    for p in range(n):
        for h in range(H):
            exact = sum(Fraction(float(w[p, j])) * Fraction(o[p, j, h]) for j in range(k))
            assert Fraction(ystar[p, h]) == exact
    # the one-token form gives the same values
    y1, s1 = oracle.combine(o[2], np.abs(o[2]), w[2])
    assert np.array_equal(y1, ystar[2])


def test_combine_one_hot_weight_and_slot_order():
    rng = np.random.default_rng(52)
    o = rng.standard_normal((1, 8, 32))
    for j in range(8):
        w = np.zeros((1, 8), np.float32)
        w[0, j] = 1.0
        y, S = oracle._combine_tokens(o, np.abs(o), w, np.ones((1, 8), bool))
        assert np.array_equal(y[0], o[0, j]) and np.array_equal(S[0], np.abs(o[0, j]))
    # a wrong pairing of weights and slots is caught: reversing the weights changes y
    w = np.arange(1, 9, dtype=np.float32)[None]
    y, _ = oracle._combine_tokens(o, np.abs(o), w, np.ones((1, 8), bool))
    yr, _ = oracle._combine_tokens(o, np.abs(o), w[:, ::-1].copy(), np.ones((1, 8), bool))
    assert not np.allclose(y, yr)


# ----------------------------------------------------------------------------- dense-MLP case
def _nvfp4_exact_x(rng, T, H, g_x):
    """bf16-representable x whose NVFP4 quantization with g_x reproduces it exactly: every
    16-block holds a +-6 and a power-of-two scale, g_x a power of two."""
    codes = rng.integers(0, 16, (T, H)).astype(np.uint8)
    codes[:, ::16] = rng.choice([7, 15], (T, H // 16))
    u = rng.integers(-3, 4, (T, H // 16))
    mag = np.array(E2M1)[codes & 7]
    val = np.where(codes & 8, -mag, mag) * np.repeat(np.exp2(u), 16, axis=1) * g_x
    x = val.astype(np.float32)
    assert np.array_equal(x.astype(np.float64), val)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return x, packed, ((u + 7) << 3).astype(np.uint8)


def _nvfp4_weights(rng, rows, K):
    c = rng.integers(0, 256, (rows, K // 2), dtype=np.uint8)
    s = ((rng.integers(-4, 5, (rows, K // 16)) + 7) << 3).astype(np.uint8)
    return c, s


@pytest.mark.parametrize("T,H,I", [(5, 64, 32), (3, 128, 48)])
def test_nvfp4_layer_reduces_to_dense_mlp(T, H, I):
    rng = np.random.default_rng(60 + H)
    g_x, g_w1, g_w2 = 2.0 ** -6, 0.25, 0.5
    x, xq_want, xsf_want = _nvfp4_exact_x(rng, T, H, g_x)
    w13, w13_sf = _nvfp4_weights(rng, 2 * I, H)
    w2, w2_sf = _nvfp4_weights(rng, H, I)
    logits = rng.standard_normal((T, 1)).astype(np.float32)
    ids, w = oracle.route_noaux(logits, np.zeros(1, np.float32), 1, 1, 1, 2.5)
    assert np.all(ids == 0) and np.all(w == np.float32(2.5))
    # numpy float64 dense MLP
    W1 = _dec_nvfp4(w13, w13_sf) * g_w1
    gate, up = x.astype(np.float64) @ W1[:I].T, x.astype(np.float64) @ W1[I:].T
    h = gate * expit(gate) * up
    g_h = float(np.float32(np.abs(h).max() / 2688.0))
    hq, hsf = oracle.quantize_nvfp4(h.astype(np.float32), g_h)
    W2 = _dec_nvfp4(w2, w2_sf) * g_w2
    o = (_dec_nvfp4(hq, hsf) * g_h) @ W2.T
    ystar = 2.5 * o
    Sabs = 2.5 * (np.abs(_dec_nvfp4(hq, hsf) * g_h) @ np.abs(W2).T)

    res = oracle.moe_layer_nvfp4(x, g_x, ids, w, T, lambda e: (w13, w13_sf, w2, w2_sf),
                                 np.array([g_w1], np.float32), np.array([g_w2], np.float32), g_h, I)
    assert np.array_equal(res["xq"], xq_want) and np.array_equal(res["xsf"], xsf_want)
    assert np.array_equal(res["g1"][:, 0, :I], gate) and np.array_equal(res["g1"][:, 0, I:], up)  # exact sums
    assert np.allclose(res["h"][:, 0], h, rtol=1e-14, atol=0)
    assert np.array_equal(res["hq"][:, 0], hq) and np.array_equal(res["hsf"][:, 0], hsf)
    assert np.all(np.abs(res["ystar"] - ystar) <= 1e-12 * Sabs)
    assert np.array_equal(res["y"], oracle.bf16_bits(ystar))
    # the layer's intermediate really is quantized: the unquantized h gives another y
    o_raw = h @ W2.T
    assert not np.allclose(2.5 * o_raw, ystar, rtol=1e-6)


def _fp8_codes(rng, shape):
    c = rng.integers(0, 0x7F, shape).astype(np.uint8)        # finite magnitudes
    return c | (rng.integers(0, 2, shape) * 0x80).astype(np.uint8)


@pytest.mark.parametrize("full_precision_h", [False, True])
def test_fp8_layer_reduces_to_dense_mlp(full_precision_h):
    rng = np.random.default_rng(70 + full_precision_h)
    T, H, I = 4, 256, 128
    xq = _fp8_codes(rng, (T, H))
    xs = rng.uniform(0.001, 0.01, (T, H // 128)).astype(np.float32)
    w13 = _fp8_codes(rng, (2 * I, H))
    w13_s = rng.uniform(1e-4, 1e-3, (2 * I // 128, H // 128)).astype(np.float32)
    w2 = _fp8_codes(rng, (H, I))
    w2_s = rng.uniform(1e-4, 1e-3, (H // 128, I // 128)).astype(np.float32)
    ids, w = oracle.route_noaux(rng.standard_normal((T, 1)).astype(np.float32), np.zeros(1, np.float32),
                                1, 1, 1, 2.5)
    X = _e4m3_torch(xq) * np.repeat(xs.astype(np.float64), 128, axis=1)
    W1 = _e4m3_torch(w13) * np.kron(w13_s.astype(np.float64), np.ones((128, 128)))
    W2 = _e4m3_torch(w2) * np.kron(w2_s.astype(np.float64), np.ones((128, 128)))
    gate, up = X @ W1[:I].T, X @ W1[I:].T
    h = gate * expit(gate) * up
    hb = h if full_precision_h else oracle.bf16_value(oracle.bf16_bits(h))
    ystar = 2.5 * (hb @ W2.T)
    Sabs = 2.5 * (np.abs(hb) @ np.abs(W2).T)
    res = oracle.moe_layer_fp8(xq, xs, ids, w, T, lambda e: (w13, w13_s, w2, w2_s), I,
                               full_precision_h=full_precision_h)
    S1 = np.abs(X) @ np.abs(W1).T
    assert np.all(np.abs(res["g1"][:, 0] - np.concatenate([gate, up], 1)) <= 1e-13 * S1)
    if full_precision_h:   # fp64 h*: equal up to the rounding of the two fp64 evaluations
        assert np.allclose(res["hb"][:, 0], hb, rtol=1e-12, atol=0)
    else:
        assert np.array_equal(res["hb"][:, 0], hb)
    assert np.all(np.abs(res["ystar"] - ystar) <= 1e-12 * Sabs)
    assert np.array_equal(res["y"], oracle.bf16_bits(ystar))
    if not full_precision_h:
        assert not np.array_equal(hb, h)                      # the bf16 rounding took place


# ----------------------------------------------------------------------------- layer invariants
def _small_nvfp4_layer(rng, T, E, H, I, k):
    x = (rng.standard_normal((T, H))).astype(np.float32)
    x = oracle.bf16_value(oracle.bf16_bits(x)).astype(np.float32)
    W = {e: (*_nvfp4_weights(rng, 2 * I, H), *_nvfp4_weights(rng, H, I)) for e in range(E)}
    logits = rng.standard_normal((T, E)).astype(np.float32)
    bias = (rng.standard_normal(E) * 0.01).astype(np.float32)
    ids, w = oracle.route_noaux(logits, bias, 2, 1, k, 2.5)
    return x, W, ids, w


def test_nvfp4_layer_token_separable_and_subset():
    rng = np.random.default_rng(80)
    T, E, H, I, k = 12, 8, 64, 32, 2
    x, W, ids, w = _small_nvfp4_layer(rng, T, E, H, I, k)
    g = np.full(E, 0.25, np.float32)
    g_x = float(np.float32(np.abs(x).max() / 2688.0))
    full = oracle.moe_layer_nvfp4(x, g_x, ids, w, T, W.__getitem__, g, g, 4096.0, I)
    perm = rng.permutation(T)
    pr = oracle.moe_layer_nvfp4(x[perm], g_x, ids[perm], w[perm], T, W.__getitem__, g, g, 4096.0, I)
    assert np.array_equal(pr["y"], full["y"][perm])
    sub = [1, 7, 10]
    sr = oracle.moe_layer_nvfp4(x, g_x, ids, w, T, W.__getitem__, g, g, 4096.0, I, tokens=sub)
    assert np.array_equal(sr["y"], full["y"][sub]) and np.array_equal(sr["ystar"], full["ystar"][sub])


def test_nvfp4_layer_capacity_drop():
    rng = np.random.default_rng(81)
    T, E, H, I, k = 10, 4, 64, 32, 2
    x, W, ids, w = _small_nvfp4_layer(rng, T, E, H, I, k)
    g = np.full(E, 0.25, np.float32)
    full = oracle.moe_layer_nvfp4(x, 0.01, ids, w, T, W.__getitem__, g, g, 4096.0, I)
    cap = 2
    dr = oracle.moe_layer_nvfp4(x, 0.01, ids, w, cap, W.__getitem__, g, g, 4096.0, I)
    _, row = oracle.dispatch(ids, E, cap)
    kept = row < cap
    assert not kept.all()
    assert np.array_equal(dr["kept"], kept)
    want, _ = oracle._combine_tokens(full["o"], full["so"], w, kept)
    assert np.array_equal(dr["ystar"], want)
