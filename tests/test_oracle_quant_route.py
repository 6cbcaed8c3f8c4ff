"""Pins for the oracle's NVFP4 quantizer, no-aux router and dispatch (CPU only)."""
import itertools

import numpy as np
import pytest
from scipy.special import expit

import oracle

E2M1_MAGS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _nearest_e2m1(a):
    """Independent rule for a non-negative magnitude: walk the midpoints."""
    c = 0
    for i in range(7):
        mid = (E2M1_MAGS[i] + E2M1_MAGS[i + 1]) / 2
        if a > mid or (a == mid and (i + 1) % 2 == 0):
            c = i + 1
    return c


# ----------------------------------------------------------------------------- quantizer
@pytest.mark.parametrize("g", [0.5, 1.0, 0.037])
def test_quantize_round_trip(g):
    rng = np.random.default_rng(20)
    rows, K = 6, 128
    codes = rng.integers(0, 16, (rows, K)).astype(np.uint8)
    codes[:, ::16] = 7  # every block holds a +6
    scode = rng.integers(0x18, 0x60, (rows, K // 16)).astype(np.uint8)  # general e4m3 scales
    sval = oracle.e4m3_table()[scode]
    # x = e2m1 * S * g formed in fp32 (each step exact: <= 6 significant bits)
    x = (oracle.e2m1_table()[codes].astype(np.float32) *
         np.repeat(sval.astype(np.float32), 16, axis=1) * np.float32(g)).astype(np.float32)
    q, sf = oracle.quantize_nvfp4(x, g)
    want_codes = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    # amax/(6g) recovers S exactly when 6g is exact; otherwise allow the neighbouring code
    if g in (0.5, 1.0):
        assert np.array_equal(sf, scode)
        assert np.array_equal(q & 0x77, want_codes & 0x77)  # -0 inputs stay -0 (sign kept)
        assert np.array_equal(q, want_codes)
    else:
        assert np.all(np.abs(sf.astype(int) - scode.astype(int)) <= 1)


def test_quantize_zero_and_saturation():
    K = 32
    x = np.zeros((3, K), np.float32)
    x[0, 5] = -0.0
    x[0, 7] = -0.0
    x[1, :16] = 1e6          # amax/(6g) = 1e6/6 > 448: scale saturates to 448
    x[1, 3] = -1e6
    x[2, 16:] = np.linspace(-5, 5, 16)
    q, sf = oracle.quantize_nvfp4(x, 1.0)
    assert sf[0, 0] == 0 and sf[0, 1] == 0
    nib = np.stack([q & 15, q >> 4], -1).reshape(3, K)
    assert nib[0, 5] == 8 and nib[0, 7] == 8 and nib[0, 0] == 0
    assert sf[1, 0] == 0x7E
    assert (nib[1, :16] == 7).sum() == 15 and nib[1, 3] == 15   # saturated at +-6
    assert sf[2, 0] == 0 and sf[2, 1] == oracle.encode_e4m3_sat(5.0 / 6.0)


def test_quantize_error_bound_random():
    rng = np.random.default_rng(21)
    x = rng.standard_normal((64, 256)).astype(np.float32)
    g = np.float32(np.abs(x).max() / 2688.0)
    q, sf = oracle.quantize_nvfp4(x, g)
    dec = oracle.nvfp4_decode(q, sf) * float(g)
    d = np.repeat(oracle.e4m3_table()[sf] * float(g), 16, axis=1)
    xr = np.abs(x) / d
    half_step = np.where(xr < 2, 0.25, np.where(xr < 4, 0.5, 1.0)) * d
    ok = (xr <= 6.0)
    assert np.all(np.abs(x - dec)[ok] <= half_step[ok] * (1 + 1e-6))
    assert np.all(np.abs(x - dec)[~ok] <= np.abs(x)[~ok] - 6 * d[~ok] + 1e-6 * d[~ok])


def test_quantize_rounding_rule_all_bf16():
    """Every finite bf16 magnitude v (g = 1) placed beside a block maximum of 6 * 448 * ...:
    the scale is fixed, so the code must be the nearest e2m1 of fl32(v * (1/d))."""
    bits = np.arange(0, 0x7F80, dtype=np.uint32)          # all finite non-negative bf16
    v = (bits << 16).view(np.float32)
    amax = np.float32(6.0 * 16.0)                            # scale code 16.0 -> d = 16
    v = v[v <= amax]
    n = len(v)
    blocks = np.zeros((n, 16), np.float32)
    blocks[:, 0] = amax
    blocks[:, 1] = v
    q, sf = oracle.quantize_nvfp4(blocks, 1.0)
    assert np.all(sf[:, 0] == oracle.encode_e4m3_sat(16.0))
    got = (q[:, 0] >> 4).astype(int)
    r = np.float32(1.0) / np.float32(16.0)
    want = np.array([_nearest_e2m1(float(np.float32(x * r))) for x in v])
    assert np.array_equal(got, want)


# ----------------------------------------------------------------------------- router
def _s_fp32(logits):
    return (1.0 / (1.0 + np.exp(-logits.astype(np.float64)))).astype(np.float32)


def _route_bruteforce(logits, bias, n_group, topk_group, top_k, rsf):
    """Enumerate every admissible choice instead of greedy selection."""
    E = logits.shape[0]
    gsz = E // n_group
    s = _s_fp32(logits)
    sb = (s + bias).astype(np.float32)
    gscore = []
    for q in range(n_group):
        vals = sorted(sb[q * gsz:(q + 1) * gsz].tolist(), reverse=True)
        gscore.append(np.float32(np.float32(vals[0]) + np.float32(vals[1])))
    # best group subset: lexicographically largest sorted score vector, then smallest indices
    best = None
    for sub in itertools.combinations(range(n_group), topk_group):
        key = (sorted([float(gscore[q]) for q in sub], reverse=True), [-q for q in sub])
        if best is None or key > best[0]:
            best = (key, sub)
    groups = best[1]
    cand = [e for e in range(E) if e // gsz in groups]
    bestk = None
    for sub in itertools.combinations(cand, top_k):
        order = sorted(sub, key=lambda e: (-float(sb[e]), e))
        key = ([float(sb[e]) for e in order], [-e for e in order])
        if bestk is None or key > bestk[0]:
            bestk = (key, order)
    ids = bestk[1]
    den = np.float32(0)
    for e in ids:
        den = np.float32(den + s[e])
    w = [np.float32(np.float32(s[e] / den) * np.float32(rsf)) for e in ids]
    return np.array(ids, np.int32), np.array(w, np.float32)


@pytest.mark.parametrize("E,ng,tg,k", [(8, 4, 2, 2), (16, 4, 2, 3), (12, 3, 1, 2), (16, 8, 4, 4)])
def test_router_bruteforce(E, ng, tg, k):
    rng = np.random.default_rng(E * 10 + k)
    T = 40
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[:5] = np.round(logits[:5])       # plant ties
    bias = (rng.standard_normal(E) * 0.01).astype(np.float32)
    ids, w = oracle.route_noaux(logits, bias, ng, tg, k, 2.5)
    for t in range(T):
        bi, bw = _route_bruteforce(logits[t], bias, ng, tg, k, 2.5)
        assert np.array_equal(ids[t], bi), t
        assert np.array_equal(w[t], bw), t


def test_router_single_group_is_plain_topk():
    rng = np.random.default_rng(30)
    T, E, k = 50, 64, 8
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[::7, ::3] = 0.25  # ties
    bias = (rng.standard_normal(E) * 0.01).astype(np.float32)
    ids, w = oracle.route_noaux(logits, bias, 1, 1, k, 1.0)
    sb = (_s_fp32(logits) + bias).astype(np.float32)
    for t in range(T):
        order = np.lexsort((np.arange(E), -sb[t].astype(np.float64)))
        assert np.array_equal(ids[t], order[:k])


def test_router_ties_lower_index_and_invariants():
    T, E = 3, 256
    logits = np.zeros((T, E), np.float32)
    bias = np.zeros(E, np.float32)
    ids, w = oracle.route_noaux(logits, bias, 8, 4, 8, 2.5)
    assert np.array_equal(ids[0], np.arange(8))         # all equal -> lowest indices, group 0
    assert np.allclose(w, 2.5 / 8)
    rng = np.random.default_rng(31)
    T = 128
    logits = rng.standard_normal((T, E)).astype(np.float32)
    bias = (rng.standard_normal(E) * 0.01).astype(np.float32)
    ids, w = oracle.route_noaux(logits, bias, 8, 4, 8, 2.5)
    for t in range(T):
        assert len(set(ids[t].tolist())) == 8
        assert len(set((ids[t] // 32).tolist())) <= 4
        # weights follow the library logistic function of the selected logits
        ref = expit(logits[t, ids[t]].astype(np.float64))
        assert np.allclose(w[t], 2.5 * ref / ref.sum(), rtol=4 * 2 ** -23, atol=0)
        assert abs(float(w[t].astype(np.float64).sum()) - 2.5) < 16 * 2 ** -23 * 2.5
        # slot order: s + bias non-increasing
        sbt = (_s_fp32(logits[t]) + bias).astype(np.float32)[ids[t]]
        assert np.all(sbt[:-1] >= sbt[1:])


# ----------------------------------------------------------------------------- dispatch
def test_dispatch_bruteforce_and_invariants():
    rng = np.random.default_rng(40)
    T, E, k = 30, 10, 3
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    for max_m in (100, 5):
        mm, row = oracle.dispatch(ids, E, max_m)
        for e in range(E):
            toks = [t for t in range(T) if e in ids[t]]
            assert mm[e] == min(len(toks), max_m)
            for rank, t in enumerate(toks):
                j = list(ids[t]).index(e)
                assert row[t, j] == rank
    mm, row = oracle.dispatch(ids, E, 1000)
    assert mm.sum() == T * k
    pairs = {(int(ids[t, j]), int(row[t, j])) for t in range(T) for j in range(k)}
    assert len(pairs) == T * k


@pytest.mark.parametrize("T,E,k,align", [(1, 8, 2, 16), (37, 16, 4, 8), (200, 256, 8, 128)])
def test_dispatch_contiguous_invariants(T, E, k, align):
    # brute force in token order: each slot takes the next free row of its expert's
    # aligned segment; segments follow each other in expert order
    rng = np.random.default_rng(T * 7 + E)
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    start, count, row = oracle.dispatch_contiguous(ids, E, align)
    want_count = np.bincount(ids.ravel(), minlength=E)
    assert np.array_equal(count, want_count)
    pos = 0
    for e in range(E):
        assert start[e] == pos and start[e] % align == 0
        pos += -(-int(want_count[e]) // align) * align
    assert start[E] == pos
    nxt = start[:E].astype(np.int64).copy()
    for t in range(T):
        for j in range(k):
            e = ids[t, j]
            assert row[t, j] == nxt[e]
            nxt[e] += 1
    assert len(np.unique(row)) == T * k


# ----------------------------------------------------------------------------- quantizer steps in exact arithmetic
def _rnd32(q):
    """Nearest IEEE binary32 value to the rational q (ties to even), subnormals included."""
    from fractions import Fraction
    if q == 0:
        return Fraction(0)
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    quantum = Fraction(2) ** (max(e, -126) - 23)
    n = a / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * quantum
    return r if q > 0 else -r


def _frac_e4m3_mag(c):
    from fractions import Fraction
    e, m = (c >> 3) & 15, c & 7
    return Fraction(m, 512) if e == 0 else Fraction(8 + m, 8) * Fraction(2) ** (e - 7)


def _nearest_e4m3_code(q):
    """Nearest finite non-negative e4m3fn code to q >= 0 (ties to the even code), saturating."""
    if q > 448:
        return 0x7E
    best = min(range(0x7F), key=lambda c: (abs(_frac_e4m3_mag(c) - q), c & 1))
    return best


def _nearest_e2m1_frac(v):
    """Nearest e2m1 code of a rational v (sign kept, ties to the code with LSB 0, |v| > 6 -> 6)."""
    from fractions import Fraction
    mags = [Fraction(x) for x in (0, 0.5, 1, 1.5, 2, 3, 4, 6)]
    a = abs(v)
    c = 7 if a > 6 else min(range(8), key=lambda i: (abs(mags[i] - a), i & 1))
    return c | (8 if v < 0 else 0)


def _quantize_block_exact(xb, g):
    """The quantizer's reading step by step, each fp32 operation rounded from the exact
    rational result: S = e4m3(fl(amax / fl(6 g))), d = fl(S g), r = fl(1 / d),
    code = e2m1(fl(x r)).  Also returns the codes the other reading, e2m1(fl(x / d)), gives."""
    from fractions import Fraction
    xs = [Fraction(float(v)) for v in xb]
    gf = Fraction(float(g))
    six_g = _rnd32(6 * gf)
    amax = max(abs(v) for v in xs)
    sc = _nearest_e4m3_code(_rnd32(amax / six_g))
    sval = _frac_e4m3_mag(sc)
    if sval == 0:
        codes = [8 if np.signbit(v) else 0 for v in xb]
        return sc, codes, codes
    d = _rnd32(sval * gf)
    r = _rnd32(1 / d)
    by_rcp = [_nearest_e2m1_frac(_rnd32(v * r)) | (8 if np.signbit(xb[i]) else 0) for i, v in enumerate(xs)]
    by_div = [_nearest_e2m1_frac(_rnd32(v / d)) | (8 if np.signbit(xb[i]) else 0) for i, v in enumerate(xs)]
    return sc, by_rcp, by_div


def _codes_of(q):
    return np.stack([q & 15, q >> 4], -1).reshape(q.shape[0], -1)


def test_quantize_multiplies_by_rounded_reciprocal():
    """Blocks where multiplying by fl(1/d) and dividing by d give different codes: the
    oracle must follow the reciprocal reading.  Among them, the block with g = 1.6267272,
    x = 36.601364 beside a block maximum that gives scale code 0x49."""
    rng = np.random.default_rng(90)
    cand_x, cand_g = [], []
    # named case: the scale code 0x49 (= 1.125 * 2^2) from a block maximum of 6 * 4.5 * g
    g0 = np.float32(1.6267272)
    xb = np.zeros(16, np.float32)
    xb[0] = np.float32(6.0 * 4.5) * g0
    xb[1] = np.float32(36.601364)
    cand_x.append(xb); cand_g.append(g0)
    # searched cases: values near e2m1 midpoints in units of d
    for _ in range(4000):
        g = np.float32(np.exp(rng.uniform(-6, 3)))
        sc = rng.integers(0x20, 0x70)
        d = np.float32(np.float32(_frac_e4m3_mag(int(sc))) * g)
        mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
        xb = (rng.choice(mids, 16) * (1 + rng.integers(-4, 5, 16) * 2.0 ** -23) * float(d)).astype(np.float32)
        xb *= np.where(rng.random(16) < 0.5, -1, 1).astype(np.float32)
        xb[0] = np.float32(6.0 * float(_frac_e4m3_mag(int(sc)))) * g
        r = np.float32(1.0) / d
        if np.any(oracle.encode_e2m1(xb * r) != oracle.encode_e2m1(xb / d)):
            cand_x.append(xb); cand_g.append(g)
        if len(cand_x) >= 24:
            break
    differ = 0
    for xb, g in zip(cand_x, cand_g):
        sc, by_rcp, by_div = _quantize_block_exact(xb, g)
        q, sf = oracle.quantize_nvfp4(xb[None], float(g))
        assert sf[0, 0] == sc, (g, xb)
        assert _codes_of(q)[0].tolist() == by_rcp, (g, xb)
        differ += by_rcp != by_div
    assert differ >= 20, "too few blocks separate the two readings"
    sc, by_rcp, by_div = _quantize_block_exact(cand_x[0], cand_g[0])
    assert sc == 0x49 and by_rcp[1] == 6 and by_div[1] == 7


def test_quantize_scale_step_exact_rational():
    """The scale code comes from fl(amax / fl(6 g)) with g a general fp32 value: checked in
    exact arithmetic over random blocks, including maxima near e4m3 midpoints."""
    rng = np.random.default_rng(91)
    for i in range(300):
        g = np.float32(np.exp(rng.uniform(-8, 4)))
        xb = (rng.standard_normal(16) * np.exp(rng.uniform(-3, 3))).astype(np.float32) * g
        if i % 3 == 0:   # block maximum at 6 g times an e4m3 midpoint
            c = int(rng.integers(0x10, 0x76))
            mid = (_frac_e4m3_mag(c) + _frac_e4m3_mag(c + 1)) / 2
            xb[int(rng.integers(16))] = np.float32(6.0 * float(mid)) * g
        sc, by_rcp, _ = _quantize_block_exact(xb, g)
        q, sf = oracle.quantize_nvfp4(xb[None], float(g))
        assert sf[0, 0] == sc, (i, g)
        assert _codes_of(q)[0].tolist() == by_rcp, (i, g)
