"""Pins for the oracle's GEMMs (CPU only): brute force in exact rationals, closed forms,
the concatenation and untouched-row invariants, scale linearity and numpy's float64
matmul as a library routine."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import datagen
import oracle

SENT = 0x7FC1  # NaN payload used as the "untouched" sentinel


def _np(t):
    return t.cpu().numpy()


def _frac_e2m1(c):
    mags = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3),
            Fraction(4), Fraction(6)]
    v = mags[c & 7]
    return -v if c & 8 else v


def _frac_e4m3(c):
    s, e, m = (c >> 7) & 1, (c >> 3) & 15, c & 7
    v = Fraction(m, 512) if e == 0 else Fraction(8 + m, 8) * Fraction(2) ** (e - 7)
    return -v if s else v


def _frac_decode_row(codes, sf, K):
    out = []
    for k in range(K):
        byte = int(codes[k // 2])
        c = (byte >> 4) if k % 2 else (byte & 15)
        out.append(_frac_e2m1(c) * _frac_e4m3(int(sf[k // 16])))
    return out


@pytest.mark.parametrize("G,M,N,K", [(1, 1, 1, 16), (2, 3, 5, 32), (3, 5, 4, 48)])
def test_masked_gemm_bruteforce_exact(G, M, N, K):
    rng = np.random.default_rng(G * 100 + K)
    a = rng.integers(0, 256, (G, M, K // 2), dtype=np.uint8)
    b = rng.integers(0, 256, (G, N, K // 2), dtype=np.uint8)
    # general e4m3 scales (not only powers of two), no NaN codes
    a_sf = rng.integers(0, 0x7F, (G, M, K // 16), dtype=np.uint8)
    b_sf = rng.integers(0, 0x7F, (G, N, K // 16), dtype=np.uint8)
    a_sf[..., 0] |= 0x80 * (rng.integers(0, 2, (G, M)).astype(np.uint8))  # some negative scales
    alpha = np.array([0.375, 2.0, -0.125][:G], np.float32)
    mm = np.array([M, M - 1, 0][:G], np.int32)
    y, s, out = oracle.gemm_nvfp4_masked(a, a_sf, b, b_sf, alpha, mm, M, N, K)
    for g in range(G):
        for m in range(M):
            if m >= mm[g]:
                assert np.isnan(y[g, m]).all()
                continue
            ar = _frac_decode_row(a[g, m], a_sf[g, m], K)
            for n in range(N):
                br = _frac_decode_row(b[g, n], b_sf[g, n], K)
                exact = Fraction(float(alpha[g])) * sum(x * z for x, z in zip(ar, br))
                absum = abs(Fraction(float(alpha[g]))) * sum(abs(x * z) for x, z in zip(ar, br))
                # fp64 sum of these terms is within K ulps of the exact value
                assert abs(Fraction(y[g, m, n]) - exact) <= Fraction(K) * Fraction(2) ** -52 * absum
                assert abs(Fraction(s[g, m, n]) - absum) <= Fraction(K) * Fraction(2) ** -52 * absum
                assert out[g, m, n] == oracle.bf16_bits(np.array([y[g, m, n]]))[0]


def test_masked_gemm_pow2_scales_exact():
    """For uniform codes with 2^u scales the fp64 sum is the exact real result (every
    product is a multiple of 2^-10 below 2^14; K=1024 sums stay below 2^53 ulps)."""
    wl = datagen.masked_gemm_workload(5, "cpu", G=2, max_m=4, N=6, K=1024, masked_m=[4, 2])
    t = {k: _np(v) for k, v in wl.tensors.items()}
    y, s, _ = oracle.gemm_nvfp4_masked(t["a"], t["a_sf"], t["b"], t["b_sf"], t["alpha"],
                                       t["masked_m"], 4, 6, 1024)
    for g in range(2):
        for m in range(int(t["masked_m"][g])):
            ar = _frac_decode_row(t["a"][g, m], t["a_sf"][g, m], 1024)
            for n in range(6):
                br = _frac_decode_row(t["b"][g, n], t["b_sf"][g, n], 1024)
                exact = Fraction(float(t["alpha"][g])) * sum(x * z for x, z in zip(ar, br))
                assert Fraction(y[g, m, n]) == exact


def test_one_hot_closed_form():
    G, M, N, K = 1, 2, 7, 64
    rng = np.random.default_rng(3)
    b = rng.integers(0, 256, (G, N, K // 2), dtype=np.uint8)
    b_sf = rng.integers(0, 0x7F, (G, N, K // 16), dtype=np.uint8)
    a = np.zeros((G, M, K // 2), np.uint8)
    a_sf = np.full((G, M, K // 16), 0x38, np.uint8)  # scale 1.0
    k0 = [5, 42]
    for m, k in enumerate(k0):
        a[0, m, k // 2] = 0x2 << (4 * (k % 2))  # code 0x2 = 1.0 at k
    gB = 0.25
    y, _, _ = oracle.gemm_nvfp4_masked(a, a_sf, b, b_sf, np.array([gB], np.float32), [M], M, N, K)
    bdec = oracle.nvfp4_decode(b[0], b_sf[0])
    for m, k in enumerate(k0):
        assert np.array_equal(y[0, m], gB * bdec[:, k])


def test_identity_closed_form():
    K = 48
    N = K
    rng = np.random.default_rng(4)
    a = rng.integers(0, 256, (1, 3, K // 2), dtype=np.uint8)
    a_sf = rng.integers(0, 0x7F, (1, 3, K // 16), dtype=np.uint8)
    b = np.zeros((1, N, K // 2), np.uint8)
    for n in range(N):
        b[0, n, n // 2] |= 0x2 << (4 * (n % 2))
    b_sf = np.full((1, N, K // 16), 0x38, np.uint8)
    _, _, out = oracle.gemm_nvfp4_masked(a, a_sf, b, b_sf, None, [3], 3, N, K)
    adec = oracle.nvfp4_decode(a[0], a_sf[0])
    # a sum starting from +0 turns -0 into +0; every other value is reproduced exactly
    assert np.array_equal(out[0], oracle.bf16_bits(adec + 0.0))


def test_concatenation_and_untouched_rows():
    wl = datagen.masked_gemm_workload(7, "cpu", G=3, max_m=8, N=32, K=128, masked_m=[8, 3, 0])
    t = {k: _np(v) for k, v in wl.tensors.items()}
    sent = np.full((3, 8, 32), SENT, np.uint16)
    y, s, out = oracle.gemm_nvfp4_masked(t["a"], t["a_sf"], t["b"], t["b_sf"], t["alpha"],
                                         t["masked_m"], 8, 32, 128, out=sent)
    for g in range(3):
        mm = int(t["masked_m"][g])
        yg, sg, og = oracle.gemm_nvfp4_masked(t["a"][g:g + 1], t["a_sf"][g:g + 1], t["b"][g:g + 1],
                                              t["b_sf"][g:g + 1], t["alpha"][g:g + 1], [mm], 8, 32, 128,
                                              out=sent[g:g + 1])
        assert np.array_equal(og[0], out[g])
        assert np.array_equal(yg[0, :mm], y[g, :mm])
        assert (out[g, mm:] == SENT).all()
    # masked_m beyond capacity is clamped; negative means empty
    _, _, o2 = oracle.gemm_nvfp4_masked(t["a"], t["a_sf"], t["b"], t["b_sf"], t["alpha"],
                                        [99, -5, 2], 8, 32, 128, out=sent)
    assert (o2[1] == SENT).all() and (o2[2, 2:] == SENT).all() and not (o2[0] == SENT).any()


def test_scale_linearity():
    wl = datagen.masked_gemm_workload(8, "cpu", G=1, max_m=4, N=16, K=256, masked_m=[4])
    t = {k: _np(v) for k, v in wl.tensors.items()}
    y1, _, _ = oracle.gemm_nvfp4_masked(t["a"], t["a_sf"], t["b"], t["b_sf"], t["alpha"], [4], 4, 16, 256)
    a_sf2 = t["a_sf"] + 8  # exponent field + 1: every 2^u scale doubles (u <= 4 stays finite)
    y2, _, _ = oracle.gemm_nvfp4_masked(t["a"], a_sf2, t["b"], t["b_sf"], t["alpha"], [4], 4, 16, 256)
    assert np.array_equal(y2, 2 * y1)


def test_masked_gemm_vs_numpy_matmul():
    rng = np.random.default_rng(9)
    G, M, N, K = 2, 9, 33, 320
    a = rng.integers(0, 256, (G, M, K // 2), dtype=np.uint8)
    b = rng.integers(0, 256, (G, N, K // 2), dtype=np.uint8)
    a_sf = rng.integers(0, 0x7F, (G, M, K // 16), dtype=np.uint8)
    b_sf = rng.integers(0, 0x7F, (G, N, K // 16), dtype=np.uint8)
    alpha = np.array([0.3, 1.7], np.float32)
    y, s, _ = oracle.gemm_nvfp4_masked(a, a_sf, b, b_sf, alpha, [M, M], M, N, K)
    for g in range(G):
        ref = float(alpha[g]) * (oracle.nvfp4_decode(a[g], a_sf[g]) @ oracle.nvfp4_decode(b[g], b_sf[g]).T)
        absref = abs(float(alpha[g])) * (np.abs(oracle.nvfp4_decode(a[g], a_sf[g])) @
                                         np.abs(oracle.nvfp4_decode(b[g], b_sf[g])).T)
        assert np.all(np.abs(y[g] - ref) <= 1e-12 * absref)
        assert np.allclose(s[g], absref, rtol=1e-12, atol=0)
    # transposed operand would fail: B rows are not A rows
    assert not np.allclose(y[0, :, :M], y[0, :, :M].T)


def test_row_dot_matches_masked():
    wl = datagen.masked_gemm_workload(10, "cpu", G=1, max_m=3, N=20, K=64, masked_m=[3])
    t = {k: _np(v) for k, v in wl.tensors.items()}
    y, s, _ = oracle.gemm_nvfp4_masked(t["a"], t["a_sf"], t["b"], t["b_sf"], t["alpha"], [3], 3, 20, 64)
    for m in range(3):
        yr, sr = oracle.nvfp4_row_dot(t["a"][0], t["a_sf"][0], m, t["b"][0], t["b_sf"][0], 64,
                                      float(t["alpha"][0]))
        assert np.array_equal(yr, y[0, m]) and np.array_equal(sr, s[0, m])


# ----------------------------------------------------------------------------- FP8 block GEMM
def test_fp8_block_constant_closed_form():
    M, N, K = 3, 256, 384
    qa = np.full((M, K), 0x38, np.uint8)  # 1.0
    qb = np.full((N, K), 0x38, np.uint8)
    sa = np.arange(1, M * (K // 128) + 1, dtype=np.float32).reshape(M, K // 128) * 0.5
    sb = np.arange(1, (N // 128) * (K // 128) + 1, dtype=np.float32).reshape(N // 128, K // 128)
    y, s = oracle.gemm_fp8_block(qa, sa, qb, sb)
    for m in range(M):
        for n in range(N):
            want = sum(128 * float(sa[m, kb]) * float(sb[n // 128, kb]) for kb in range(K // 128))
            assert y[m, n] == want and s[m, n] == want


def test_fp8_block_vs_numpy_and_rows():
    rng = np.random.default_rng(11)
    M, N, K = 5, 256, 256
    qa = rng.integers(0, 0x7F, (M, K), dtype=np.uint8) | (rng.integers(0, 2, (M, K)) * 0x80).astype(np.uint8)
    qb = rng.integers(0, 0x7F, (N, K), dtype=np.uint8) | (rng.integers(0, 2, (N, K)) * 0x80).astype(np.uint8)
    sa = rng.uniform(0.01, 2, (M, K // 128)).astype(np.float32)
    sb = rng.uniform(0.01, 2, (N // 128, K // 128)).astype(np.float32)
    t = oracle.e4m3_table()
    adec = t[qa] * np.repeat(sa.astype(np.float64), 128, axis=1)
    bdec = t[qb] * np.repeat(np.repeat(sb.astype(np.float64), 128, axis=0), 128, axis=1)
    y, s = oracle.gemm_fp8_block(qa, sa, qb, sb)
    ref = adec @ bdec.T
    assert np.all(np.abs(y - ref) <= 1e-12 * (np.abs(adec) @ np.abs(bdec).T))
    y2, _ = oracle.gemm_fp8_block(qa, sa, qb, sb, rows=[4, 1])
    assert np.array_equal(y2, y[[4, 1]])
    # dense-activation form with bf16-valued activations
    yd, _ = oracle.gemm_dense_fp8w(adec[:2], qb, sb)
    assert np.allclose(yd, ref[:2], rtol=1e-12, atol=1e-9)


def test_fp8_block_bruteforce_tiny():
    rng = np.random.default_rng(12)
    M, N, K = 2, 128, 128
    qa = rng.integers(0, 0x7F, (M, K), dtype=np.uint8)
    qb = rng.integers(0x80, 0xFF, (N, K), dtype=np.uint8)
    sa = np.array([[0.75], [3.0]], np.float32)
    sb = np.array([[0.125]], np.float32)
    y, _ = oracle.gemm_fp8_block(qa, sa, qb, sb)
    for m in range(M):
        for n in (0, 77, 127):
            exact = sum(_frac_e4m3(int(qa[m, k])) * _frac_e4m3(int(qb[n, k])) for k in range(K))
            exact *= Fraction(float(sa[m, 0])) * Fraction(float(sb[0, 0]))
            assert Fraction(y[m, n]) == exact


def test_swiglu_closed_forms():
    I = 5
    gu = np.array([[0.0, 1.0, -2.0, 30.0, -40.0, 3.0, 3.0, 3.0, 3.0, 3.0]])
    h = oracle.swiglu(gu, I)
    from scipy.special import expit
    g = gu[0, :I]
    want = g * expit(g) * 3.0  # library logistic function
    assert np.allclose(h[0], want, rtol=1e-15, atol=0)
    assert h[0, 0] == 0.0
    assert abs(h[0, 3] - 90.0) < 1e-9 and abs(h[0, 4]) < 1e-15  # silu(30) ~ 30, silu(-40) ~ 0
    # gate/up swap must change the result
    h2 = oracle.swiglu(np.concatenate([gu[:, I:], gu[:, :I]], axis=1), I)
    assert not np.array_equal(h, h2)


# ----------------------------------------------------------------------------- W4A16 GEMV
def _frac_bf16(bits):
    s, e, m = (bits >> 15) & 1, (bits >> 7) & 0xFF, bits & 0x7F
    v = Fraction(m, 128) * Fraction(2) ** -126 if e == 0 else Fraction(128 + m, 128) * Fraction(2) ** (e - 127)
    return -v if s else v


def _random_bf16_bits(rng, shape):
    # finite values over a wide exponent range, subnormals included, no NaN / inf
    e = rng.integers(0, 200, shape).astype(np.uint16)
    m = rng.integers(0, 128, shape).astype(np.uint16)
    s = rng.integers(0, 2, shape).astype(np.uint16)
    return (s << 15) | (e << 7) | m


@pytest.mark.parametrize("M,N,K", [(1, 3, 32), (2, 4, 64)])
def test_gemv_w4a16_bruteforce_exact(M, N, K):
    rng = np.random.default_rng(M * 1000 + K)
    x = _random_bf16_bits(rng, (M, K))
    x[:, : K // 2] = (x[:, : K // 2] & 0x807F) | (rng.integers(120, 135, (M, K // 2)).astype(np.uint16) << 7)
    w = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    w_sf = rng.integers(0, 0x7F, (N, K // 16), dtype=np.uint8)
    w_sf[:, 0] |= 0x80  # a negative scale per row
    g = -0.375
    y, s = oracle.gemv_nvfp4_w4a16(x, w, w_sf, g)
    for n in range(N):
        wr = _frac_decode_row(w[n], w_sf[n], K)
        for m in range(M):
            prods = [_frac_bf16(int(x[m, k])) * wr[k] for k in range(K)]
            exact = Fraction(g) * sum(prods)
            exact_abs = abs(Fraction(g)) * sum(abs(p) for p in prods)
            bound = K * 2.0 ** -52 * float(exact_abs)
            assert abs(y[m, n] - float(exact)) <= bound, (m, n)
            assert abs(s[m, n] - float(exact_abs)) <= bound, (m, n)


def test_gemv_w4a16_single_element_closed_form():
    # x is zero except x[0, k0] = -1.5: y[0, n] = g * (-1.5) * e2m1(code[n, k0]) * e4m3(sf[n, k0 / 16])
    rng = np.random.default_rng(7)
    N, K, k0, g = 6, 96, 37, 0.25
    x = np.zeros((1, K), np.uint16)
    x[0, k0] = 0xBFC0
    w = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    w_sf = rng.integers(0, 0x7F, (N, K // 16), dtype=np.uint8)
    y, s = oracle.gemv_nvfp4_w4a16(x, w, w_sf, g)
    for n in range(N):
        code = (int(w[n, k0 // 2]) >> 4) & 15  # k0 odd: high nibble
        want = float(Fraction(g) * Fraction(-3, 2) * _frac_e2m1(code) * _frac_e4m3(int(w_sf[n, k0 // 16])))
        assert y[0, n] == want and s[0, n] == abs(want)


def test_gemv_w4a16_equals_w4a4_on_nvfp4_activations():
    # activations that are exactly NVFP4 values (e2m1 * e4m3 has at most 6 significant bits,
    # so bf16 holds them): the W4A16 GEMV equals the NVFP4 x NVFP4 row dot
    rng = np.random.default_rng(11)
    N, K = 9, 256
    a = rng.integers(0, 256, (1, K // 2), dtype=np.uint8)
    a_sf = rng.integers(0x28, 0x48, (1, K // 16), dtype=np.uint8)
    w = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    w_sf = rng.integers(0, 0x7F, (N, K // 16), dtype=np.uint8)
    xa = oracle.nvfp4_decode(a, a_sf)
    x_bits = oracle.bf16_bits(xa)
    assert np.array_equal(oracle.bf16_value(x_bits), xa)
    y, s = oracle.gemv_nvfp4_w4a16(x_bits, w, w_sf, 0.5)
    y4, s4 = oracle.nvfp4_row_dot(a, a_sf, 0, w, w_sf, K, alpha=0.5)
    assert np.allclose(y[0], y4, rtol=1e-13, atol=1e-12) and np.allclose(s[0], s4, rtol=1e-13)


def test_rows_form_matches_row_dot():
    # the row-subset form used for token subsets gives the row dot's sums bit for bit
    rng = np.random.default_rng(13)
    K, nb = 96, 11
    a = rng.integers(0, 256, (7, K // 2), dtype=np.uint8)
    a_sf = rng.integers(0, 0x7F, (7, K // 16), dtype=np.uint8)
    b = rng.integers(0, 256, (nb, K // 2), dtype=np.uint8)
    b_sf = rng.integers(0, 0x7F, (nb, K // 16), dtype=np.uint8)
    rows = [6, 0, 3, 3]
    y, s = oracle.gemm_nvfp4_rows(a, a_sf, rows, b, b_sf, K, alpha=-0.375)
    for i, r in enumerate(rows):
        yr, sr = oracle.nvfp4_row_dot(a, a_sf, r, b, b_sf, K, alpha=-0.375)
        assert np.array_equal(y[i], yr) and np.array_equal(s[i], sr)
