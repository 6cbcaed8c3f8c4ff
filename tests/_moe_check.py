"""Stage-by-stage checks of a GPU MoE layer run against the oracle (teacher forcing).

Each stage is compared with the oracle applied to the GPU's own inputs to that stage: a
GPU that accumulates in fp32 may land on the other side of a bf16 / e2m1 rounding
boundary than the fp64 oracle, and one flipped code changes everything downstream.
Integer stages (gathered codes, scale bytes, requantized h) are bit-exact.  The checks
run per expert over every checked token routed to it, so a few hundred tokens of a
full-size layer cost one pass over each touched expert's weights.

SwiGLU tolerance (derived): with the GEMM1 outputs inside t_g = 1e-5 S_g + ulp32(g),
t_u = 1e-5 S_u + ulp32(u), and |silu'| <= 1.1,
    |h_gpu - h*| <= 1.1 (|u| + t_u) t_g + |silu(g)| t_u + 8 ulp32(h*)
(+ 1 bf16 ulp when h is stored as bf16).

The end-to-end comparison with the oracle's own chain (moe_layer_*) is reported, not
gated: it counts the y elements inside the tolerance against the oracle's y*.
"""
import numpy as np
from scipy.special import expit

import oracle
from _helpers import assert_within, bf16_from_bits_np, log, ulp_bf16, ulp_f32, within


def swiglu_tol(g, u, Sg, Su, h, xg=0.0, xu=0.0):
    """h tolerance from the GEMM1 tolerances of gate and up (xg, xu: their extra terms)."""
    tg = 1e-5 * Sg + ulp_f32(g) + xg
    tu = 1e-5 * Su + ulp_f32(u) + xu
    return 1.1 * (np.abs(u) + tu) * tg + np.abs(g * expit(g)) * tu + 8 * ulp_f32(h)


def fp8_mfma_extra(qa, sa, qb, sb):
    """Extra GEMM1 allowance for the scaled fp8 MFMA, [len(qa), len(qb)].  The instruction
    sums each group of 8 consecutive K products aligned to the group's largest product and
    drops the bits below 2^-14 of it (measured on gfx950: 1 + 2^-14 survives, 1 + 2^-15
    and seven 2^-18 products beside a 1 are lost, always toward -inf), so a group loses
    less than 8 * 2^-14 of its largest |product|.  That product is at most max|a| * max|b|
    over the group, and the block's two scales multiply the group sums: the bound is
    2^-11 * sum_blocks |sa * sb| * sum_groups max|a| * max|b|.  qa [M, K] and qb [N, K]
    e4m3 codes, sa [M, K/128], sb [N/128, K/128]."""
    mag = np.abs(oracle.e4m3_table())
    M, K = qa.shape
    N = qb.shape[0]
    # |e4m3| grows with the code's low 7 bits, so the group maxima come from the bytes
    amax = mag[(np.asarray(qa) & 0x7F).reshape(M, K // 8, 8).max(-1)]
    bmax = mag[(np.asarray(qb) & 0x7F).reshape(N, K // 8, 8).max(-1)]
    out = np.zeros((M, N))
    for b in range(K // 128):
        g = slice(16 * b, 16 * b + 16)
        out += (amax[:, g] @ bmax[:, g].T) * np.abs(np.asarray(sa, np.float64)[:, b])[:, None] \
            * np.repeat(np.abs(np.asarray(sb, np.float64)[:, b]), 128)[None, :N]
    return 2.0 ** -11 * out


def tokens_subset(T, n, seed, row=None, max_m=None, n_deep=0):
    """Sorted token ids: n drawn from the seed (all if n is None or >= T), plus n_deep
    tokens with a slot past the first 256 rows of its expert (a later M tile)."""
    if n is None or n >= T:
        toks = set(range(T))
    else:
        toks = set(np.random.default_rng(seed).choice(T, size=n, replace=False).tolist())
    if n_deep:
        deep = np.flatnonzero(((row >= 256) & (row < max_m)).any(axis=1))
        assert len(deep) >= n_deep, "workload has too few rows past 256"
        toks |= set(deep[np.linspace(0, len(deep) - 1, n_deep).astype(int)].tolist())
    return np.array(sorted(toks))


def _slots_by_expert(ids, row, max_m, toks):
    by_e = {}
    for p, t in enumerate(toks):
        for j in range(ids.shape[1]):
            if row[t, j] < max_m:
                by_e.setdefault(int(ids[t, j]), []).append((p, j, int(row[t, j])))
    return by_e


def _check_g1(g1_gpu, gu, S1, what, extra=None):
    """GEMM1 debug stage: the GPU's fp32 gate/up sums against the oracle's, 1e-5 S + 1 fp32
    ulp.  With `extra` (the fp8 MFMA's allowance) every sum must lie within that bound plus
    `extra`, and at least 99% within the bound alone."""
    if g1_gpu is None:
        return
    g = g1_gpu.astype(np.float64)
    if extra is None:
        assert_within(g, gu, S1, what, ulp=ulp_f32)
        return
    assert_within(g, gu, S1, what, ulp=ulp_f32, extra=extra)
    frac = within(g, gu, S1, ulp=ulp_f32).mean()
    assert frac >= 0.99, f"{what}: only {frac * 100:.2f}% of the sums within 1e-5 S + 1 ulp"


def check_nvfp4_layer(*, x, g_x, ids, w, row, max_m, I, weights, g_w13, g_w2, g_h, gathered, h_pre,
                      y_bits, toks, what, e2e_tokens=0, g1=None):
    """gathered(e) -> (a codes [max_m, H/2], a scales, h codes [max_m, I/2], h scales) from the
    GPU workspace; h_pre(e) -> GPU fp32 pre-quantization h [max_m, I]; weights(e) -> the
    logical (stacked) W13 and W2 codes/scales; y_bits [T, H] bf16 bits of the GPU output;
    g1(e) -> the GPU's fp32 GEMM1 debug output [max_m, 2I] (gate | up), or None."""
    xq, xsf = oracle.quantize_nvfp4(np.asarray(x, np.float32)[toks], g_x)
    H = xq.shape[1] * 2
    n, k = len(toks), ids.shape[1]
    o = np.zeros((n, k, H)); so = np.zeros((n, k, H)); kept = np.zeros((n, k), bool)
    by_e = _slots_by_expert(ids, row, max_m, toks)
    for i, (e, sl) in enumerate(sorted(by_e.items())):
        a, a_sf, hc, hsf = gathered(e)
        w13, w13_sf, w2, w2_sf = weights(e)
        pos = np.array([p for p, _, _ in sl]); js = np.array([j for _, j, _ in sl])
        rows = np.array([r for _, _, r in sl])
        assert np.array_equal(a[rows], xq[pos]) and np.array_equal(a_sf[rows], xsf[pos]), \
            f"{what}: quantized x rows of expert {e}"
        gu, S1 = oracle.gemm_nvfp4_rows(a, a_sf, rows, w13, w13_sf, H, float(g_w13[e]) * float(g_x))
        _check_g1(None if g1 is None else g1(e)[rows], gu, S1, f"{what}: GEMM1 of expert {e}")
        g, u = gu[:, :I], gu[:, I:]
        hstar = oracle.swiglu(gu, I)
        tol = swiglu_tol(g, u, S1[:, :I], S1[:, I:], hstar)
        hg = h_pre(e)[rows].astype(np.float64)
        err = np.abs(hg - hstar)
        assert np.all(err <= tol), f"{what}: h of expert {e}: max excess {np.max(err - tol)}"
        hq, hs = oracle.quantize_nvfp4(h_pre(e)[rows], g_h)
        assert np.array_equal(hc[rows], hq) and np.array_equal(hsf[rows], hs), f"{what}: requantized h, expert {e}"
        oe, se = oracle.gemm_nvfp4_rows(hc, hsf, rows, w2, w2_sf, I, float(g_w2[e]) * float(g_h))
        o[pos, js], so[pos, js], kept[pos, js] = oe, se, True
        if i % 32 == 31:
            log(f"  {what}: {i + 1} of {len(by_e)} experts checked")
    ystar, S = oracle._combine_tokens(o, so, np.asarray(w)[toks], kept)
    yb = bf16_from_bits_np(y_bits[toks])
    for p in np.flatnonzero(~kept.any(axis=1)):
        assert np.all(yb[p] == 0), f"{what}: token {toks[p]} fully dropped must give y = 0"
    assert_within(yb, ystar, S, f"{what}: y")
    log(f"{what}: {n} tokens, {len(by_e)} experts checked stage by stage")
    if e2e_tokens:
        sub = toks[:e2e_tokens]
        ref = oracle.moe_layer_nvfp4(x, g_x, ids, w, max_m, weights, g_w13, g_w2, g_h, I, tokens=sub)
        _report_e2e(what, y_bits[sub], ref)


def check_fp8_layer(*, xq, xs, ids, w, row, max_m, I, weights, gathered, h_planes, y_bits, toks, what,
                    f32h=False, o_gpu=None, e2e_tokens=0, g1=None):
    """gathered(e) -> (the token of each expert row [max_m], its scales [max_m, H/128]);
    h_planes(e) -> GPU bf16
    bits [max_m, planes * I]; weights(e) -> (w13, w13 scales, w2, w2 scales).  With f32h
    the intermediate is bf16 hi + lo: h is checked against the unrounded SwiGLU, GEMM2 and
    the combine against the oracle on hi + lo, y also against the oracle's whole layer on
    the unrounded h with the h tolerance carried through W2, and the GEMM2 output (o_gpu)
    must sit far closer to the unrounded-h result than a bf16 h does."""
    H = xq.shape[1]
    n, k = len(toks), ids.shape[1]
    o = np.zeros((n, k, H)); so = np.zeros((n, k, H)); kept = np.zeros((n, k), bool)
    if f32h:
        ox = np.zeros((n, k, H)); sx = np.zeros((n, k, H)); px = np.zeros((n, k, H))
        err2 = {"split": 0.0, "bf16": 0.0}
    by_e = _slots_by_expert(ids, row, max_m, toks)
    for i, (e, sl) in enumerate(sorted(by_e.items())):
        a_tok, a_s = gathered(e)
        w13, w13_s, w2, w2_s = weights(e)
        pos = np.array([p for p, _, _ in sl]); js = np.array([j for _, j, _ in sl])
        rows = np.array([r for _, _, r in sl])
        assert np.array_equal(a_tok[rows], toks[pos]) and np.array_equal(a_s[rows], xs[toks[pos]]), \
            f"{what}: expert rows of expert {e}"
        gu, S1 = oracle.gemm_fp8_block(xq, xs, w13, w13_s, rows=toks[pos])
        x1 = fp8_mfma_extra(xq[toks[pos]], xs[toks[pos]], w13, w13_s)
        _check_g1(None if g1 is None else g1(e)[rows], gu, S1, f"{what}: GEMM1 of expert {e}", extra=x1)
        g, u = gu[:, :I], gu[:, I:]
        hstar = oracle.swiglu(gu, I)
        hb = h_planes(e)[rows]
        if f32h:
            tol_h = swiglu_tol(g, u, S1[:, :I], S1[:, I:], hstar, x1[:, :I], x1[:, I:])
            tol = tol_h + 2.0 ** -17 * np.abs(hstar)
            hv = bf16_from_bits_np(hb[:, :I]) + bf16_from_bits_np(hb[:, I:])
        else:
            tol = swiglu_tol(g, u, S1[:, :I], S1[:, I:], hstar, x1[:, :I], x1[:, I:]) + ulp_bf16(hstar)
            hv = bf16_from_bits_np(hb)
        err = np.abs(hv - hstar)
        assert np.all(err <= tol), f"{what}: h of expert {e}: max excess {np.max(err - tol)}"
        oe, se = oracle.gemm_dense_fp8w(hv, w2, w2_s)
        o[pos, js], so[pos, js], kept[pos, js] = oe, se, True
        if f32h:
            oxe, sxe = oracle.gemm_dense_fp8w(hstar, w2, w2_s)
            pxe, _ = oracle.gemm_dense_fp8w(tol, w2 & 0x7F, np.abs(w2_s))   # |W2| codes, |scales|
            ox[pos, js], sx[pos, js], px[pos, js] = oxe, sxe, np.abs(pxe)
            ob, _ = oracle.gemm_dense_fp8w(oracle.bf16_value(oracle.bf16_bits(hstar)), w2, w2_s)
            err2["split"] += float(np.sum((o_gpu(e)[rows] - oxe) ** 2))
            err2["bf16"] += float(np.sum((ob - oxe) ** 2))
        if i % 32 == 31:
            log(f"  {what}: {i + 1} of {len(by_e)} experts checked")
    wt = np.asarray(w)[toks]
    ystar, S = oracle._combine_tokens(o, so, wt, kept)
    yb = bf16_from_bits_np(y_bits[toks])
    assert_within(yb, ystar, S, f"{what}: y")
    if f32h:
        yx, Sxx = oracle._combine_tokens(ox, sx, wt, kept)
        carry, _ = oracle._combine_tokens(px, px, np.abs(wt), kept)
        assert_within(yb, yx, Sxx + carry / 1e-5, f"{what}: y against the unrounded h")
        ratio = (err2["split"] / err2["bf16"]) ** 0.5
        log(f"{what}: GEMM2 rms error against the unrounded h, hi/lo planes / bf16 h = {ratio:.4f}")
        assert ratio < 0.05, f"the hi/lo intermediate is not much closer to the unrounded h ({ratio:.3f})"
    log(f"{what}: {n} tokens, {len(by_e)} experts checked stage by stage")
    if e2e_tokens:
        sub = toks[:e2e_tokens]
        ref = oracle.moe_layer_fp8(xq, xs, ids, w, max_m, weights, I, tokens=sub, full_precision_h=f32h)
        _report_e2e(what, y_bits[sub], ref)


def _report_e2e(what, y_bits, ref):
    yb = bf16_from_bits_np(y_bits)
    ok = within(yb, ref["ystar"], ref["S"])
    norm = np.abs(yb - ref["ystar"]) / (1e-5 * ref["S"] + ulp_bf16(ref["ystar"]))
    log(f"{what}: end to end against the oracle's own chain ({len(yb)} tokens): "
        f"{ok.mean() * 100:.3f}% of y within tolerance, max normalized error {norm.max():.3g}, "
        f"bf16 bits equal {np.mean(y_bits == ref['y']) * 100:.3f}%")
    assert np.all(np.isfinite(yb))
