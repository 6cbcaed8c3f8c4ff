"""GPU parity of the NVFP4 grouped GEMMs against the oracle (element by element on
small cases, sampled rows at the workloads' full sizes)."""
import numpy as np
import pytest
import torch

import datagen
import oracle
from _helpers import (SENT_BF16, SENT_F32, assert_within, bf16_from_bits_np, bf16_tensor_bits, log,
                      np_, sentinel_bf16, sentinel_f32, ulp_f32)

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0") if torch.cuda.is_available() else None


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import fp8_grouped_gemm_nvfp4_amd as mxg
    mxg.lib()


def _mxg():
    import fp8_grouped_gemm_nvfp4_amd as mxg
    return mxg


def _run_masked(t, max_m, N, out_dtype=torch.bfloat16, cu_limit=0):
    G = t["a"].shape[0]
    if out_dtype == torch.bfloat16:
        out = sentinel_bf16((G, max_m, N), DEV)
    else:
        out = sentinel_f32((G, max_m, N), DEV)
    _mxg().mx_grouped_gemm_masked(t["a"], t["a_sf"], t["b"], t["b_sf"], t.get("alpha"), t["masked_m"], out,
                                  cu_limit=cu_limit)
    torch.cuda.synchronize()
    return out


def _check_masked(t, out, max_m, N, K, what):
    h = {k: np_(v) for k, v in t.items() if v is not None}
    mm = np.clip(h["masked_m"], 0, max_m)
    y, s, _ = oracle.gemm_nvfp4_masked(h["a"], h["a_sf"], h["b"], h["b_sf"], h.get("alpha"), h["masked_m"],
                                       max_m, N, K)
    if out.dtype == torch.bfloat16:
        bits = bf16_tensor_bits(out)
        vals = bf16_from_bits_np(bits)
        sent, ulp = SENT_BF16, None
    else:
        bits = np_(out.view(torch.int32)).view(np.uint32)
        vals = np_(out).astype(np.float64)
        sent, ulp = SENT_F32, ulp_f32
    for g in range(len(mm)):
        m = int(mm[g])
        assert (bits[g, m:] == sent).all(), f"{what}: group {g} rows >= masked_m={m} were written"
        if m:
            kw = {} if ulp is None else {"ulp": ulp}
            assert_within(vals[g, :m], y[g, :m], s[g, :m], f"{what} group {g}", **kw)


@pytest.mark.parametrize("seed", [1000, 1001, 1002])
def test_masked_gemm_g4_m64_n512_k1024(seed):
    log(f"masked NVFP4 GEMM G=4 max_m=64 N=512 K=1024 seed={seed}")
    wl = datagen.masked_gemm_workload(seed, DEV)
    out = _run_masked(wl.tensors, 64, 512)
    _check_masked(wl.tensors, out, 64, 512, 1024, f"seed {seed}")


@pytest.mark.parametrize("G,max_m,N,K,mm", [
    (4, 64, 512, 1024, [0, 64, 1, 63]),
    (3, 64, 512, 1024, [99, -3, 17]),        # clamped to [0, max_m]
    (1, 1, 16, 64, [1]),                     # smallest case, one K step
    (2, 37, 520, 256, [37, 20]),             # M and N tails
    (2, 200, 136, 128, [200, 129]),          # several 128-row tiles, ragged
    (5, 8, 4096, 512, [1, 0, 8, 3, 1]),      # decode-shaped (16-row tiles)
    (2, 16, 264, 192, [16, 5]),
    # decode-shaped kernel (row capacity <= 32, K % 512 == 0)
    (6, 16, 520, 1024, [1, 16, 0, 7, 15, 2]),
    (4, 32, 384, 512, [17, 32, 16, 31]),
    (3, 8, 4096, 7168, [1, 8, 3]),
    (2, 1, 64, 2048, [1, 1]),
    # decode-shaped kernel (row capacity <= 8)
    (3, 8, 200, 1024, [8, 1, 5]),            # N tail inside a 128-column unit
    (4, 8, 48, 4096, [2, 0, 8, 7]),          # N below one 128-column unit
    # weight-streaming kernel (row capacity > 32, N % 128 == 0, K % 128 == 0)
    (3, 300, 256, 384, [300, 257, 31]),      # two 256-row M tiles, ragged
    (2, 96, 384, 128, [96, 65]),             # one K step, rows across a 64-row boundary
    (4, 40, 128, 256, [33, 0, 40, 1]),       # empty group, 1-row group
])
def test_masked_gemm_edges(G, max_m, N, K, mm):
    log(f"masked NVFP4 GEMM edge G={G} max_m={max_m} N={N} K={K} masked_m={mm}")
    wl = datagen.masked_gemm_workload(7, DEV, G=G, max_m=max_m, N=N, K=K, masked_m=mm)
    out = _run_masked(wl.tensors, max_m, N)
    _check_masked(wl.tensors, out, max_m, N, K, "edge")


def test_masked_gemm_general_scales_fp32_out_and_poison():
    """General e4m3 scales (including subnormal codes and negative scales), fp32 output,
    and A rows beyond masked_m poisoned with NaN scales (never read)."""
    log("masked NVFP4 GEMM general scales / fp32 out / poisoned padding")
    g = datagen.generator(11, DEV)
    G, max_m, N, K = 3, 48, 200, 320
    t = dict(a=datagen.uniform_bytes(g, (G, max_m, K // 2), DEV),
             a_sf=torch.randint(0, 0x7F, (G, max_m, K // 16), generator=g, device=DEV, dtype=torch.int32).to(torch.uint8),
             b=datagen.uniform_bytes(g, (G, N, K // 2), DEV),
             b_sf=(torch.randint(0, 0x7F, (G, N, K // 16), generator=g, device=DEV, dtype=torch.int32)
                   | (torch.randint(0, 2, (G, N, K // 16), generator=g, device=DEV, dtype=torch.int32) << 7)).to(torch.uint8),
             masked_m=torch.tensor([48, 30, 5], dtype=torch.int32, device=DEV),
             alpha=torch.tensor([0.37, 1.0, 3.5e-3], dtype=torch.float32, device=DEV))
    t["a_sf"][1, 30:] = 0x7F
    t["a_sf"][2, 5:] = 0xFF
    for dt in (torch.float32, torch.bfloat16):
        out = _run_masked(t, max_m, N, out_dtype=dt)
        vals = np_(out.float())
        for gg, m in enumerate([48, 30, 5]):
            assert np.isfinite(vals[gg, :m]).all()
        _check_masked(t, out, max_m, N, K, f"general scales {dt}")


@pytest.mark.parametrize("max_m,K", [(16, 1024), (8, 1024), (48, 512), (272, 640)])
def test_masked_gemm_fp32_out(max_m, K):
    log(f"masked NVFP4 GEMM fp32 output max_m={max_m} K={K}")
    wl = datagen.masked_gemm_workload(23, DEV, G=3, max_m=max_m, N=256, K=K, masked_m=[max_m, 1, max_m - 3])
    out = _run_masked(wl.tensors, max_m, 256, out_dtype=torch.float32)
    _check_masked(wl.tensors, out, max_m, 256, K, "fp32 out")


def test_masked_gemm_cu_limit_and_determinism():
    log("masked NVFP4 GEMM cu_limit grid-stride path and run-to-run determinism")
    wl = datagen.masked_gemm_workload(21, DEV, G=8, max_m=130, N=384, K=512)
    o1 = _run_masked(wl.tensors, 130, 384)
    o2 = _run_masked(wl.tensors, 130, 384)
    o3 = _run_masked(wl.tensors, 130, 384, cu_limit=3)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(o1.view(torch.int16), o3.view(torch.int16))
    _check_masked(wl.tensors, o3, 130, 384, 512, "cu_limit")
    wl = datagen.masked_gemm_workload(22, DEV, G=8, max_m=16, N=384, K=1024)
    o1 = _run_masked(wl.tensors, 16, 384)
    o2 = _run_masked(wl.tensors, 16, 384, cu_limit=2)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    _check_masked(wl.tensors, o2, 16, 384, 1024, "cu_limit skinny")


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_masked_gemm_item_transitions(out_dtype):
    """Groups whose row counts give each MFMA wave of the streaming kernel every count of
    valid 16-row groups (0 to 4) and a second M tile, run with 1 and 2 CUs so that one
    workgroup chains many items of different shapes (each item re-reads its first step's
    fragments and runs its own specialised loop).  Every output against the oracle, and
    bit-identical across CU limits."""
    mm = [1, 16, 17, 48, 49, 64, 65, 113, 129, 193, 256, 257, 300, 0]
    G, max_m, N, K = len(mm), 300, 256, 384
    log(f"masked NVFP4 GEMM item transitions G={G} max_m={max_m} N={N} K={K} {out_dtype}")
    wl = datagen.masked_gemm_workload(31, DEV, G=G, max_m=max_m, N=N, K=K, masked_m=mm)
    outs = [_run_masked(wl.tensors, max_m, N, out_dtype=out_dtype, cu_limit=cl) for cl in (1, 2, 0)]
    view = torch.int16 if out_dtype == torch.bfloat16 else torch.int32
    for o in outs[1:]:
        assert torch.equal(outs[0].view(view), o.view(view)), "result depends on the CU limit"
    _check_masked(wl.tensors, outs[0], max_m, N, K, "item transitions")


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_masked_gemm_balanced_tiles(out_dtype):
    """K >= 4096: groups above 256 rows split into M tiles of one height (257 rows: 144 +
    113; 600: 208 + 208 + 184; 3841: tiles of 256 and a last one of 1).  Every output
    against the oracle, bit-identical across CU limits, and the rows past masked_m left
    untouched."""
    mm = [257, 300, 432, 511, 513, 600, 256, 3841, 0]
    G, max_m, N, K = len(mm), 3856, 128, 4096
    log(f"masked NVFP4 GEMM balanced M tiles G={G} max_m={max_m} N={N} K={K} {out_dtype}")
    wl = datagen.masked_gemm_workload(37, DEV, G=G, max_m=max_m, N=N, K=K, masked_m=mm)
    outs = [_run_masked(wl.tensors, max_m, N, out_dtype=out_dtype, cu_limit=cl) for cl in (3, 0)]
    view = torch.int16 if out_dtype == torch.bfloat16 else torch.int32
    assert torch.equal(outs[0].view(view), outs[1].view(view)), "result depends on the CU limit"
    _check_masked(wl.tensors, outs[0], max_m, N, K, "balanced tiles")


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_masked_gemm_decode_many_groups(out_dtype):
    """Row capacity 8 with 256 groups (valid rows 0..8), an N tail inside a 16-column
    group, and the same bits whatever the grid."""
    G, max_m, N, K = 256, 8, 1048, 2048
    log(f"masked NVFP4 GEMM decode shape, many groups G={G} max_m={max_m} N={N} K={K} {out_dtype}")
    gen = torch.Generator().manual_seed(77)
    mm = torch.randint(0, max_m + 1, (G,), generator=gen).to(torch.int32)
    mm[:4] = torch.tensor([8, 4, 5, 0], dtype=torch.int32)
    wl = datagen.masked_gemm_workload(1077, DEV, G=G, max_m=max_m, N=N, K=K, masked_m=mm.tolist())
    outs = []
    for cu in (0, 3):
        out = _run_masked(wl.tensors, max_m, N, out_dtype=out_dtype, cu_limit=cu)
        outs.append(out)
        _check_masked(wl.tensors, out, max_m, N, K, f"decode many groups cu_limit={cu}")
    v = [np_(o.view(torch.int16 if out_dtype == torch.bfloat16 else torch.int32)) for o in outs]
    assert np.array_equal(v[0], v[1]), "result depends on the grid"


@pytest.mark.parametrize("path", ["one_launch", "two_calls"])
def test_decode_gemm1_full_size(path):
    """Decode-shaped MoE GEMM1 at its full size: 256 experts, 8 tokens top-8, K=7168,
    N=4096 (gate and up stacked): dispatch, on-the-fly NVFP4 quantization of the bf16
    activations into the masked layout, then the masked GEMM with bf16 output.  The
    one-launch dispatch + quantize-gather is the path the benchmark times; the two-call
    path is the general one.  Both are checked against the oracle: masked_m, row, every
    dispatched code and scale byte bit-exact, every valid output row within tolerance."""
    log(f"decode GEMM1 E=256 T=8 top8 H=7168 N=4096, dispatch + quantize-gather {path}")
    mxg = _mxg()
    wl = datagen.decode_gemm1_workload(1001, DEV)
    t, s = wl.tensors, wl.scalars
    E, T, H, N, max_m = 256, 8, 7168, 4096, 8
    if path == "one_launch":
        masked_m, row, a, a_sf = mxg.moe_dispatch_quantize_gather_nvfp4(t["x"], s["g_x"], t["ids"], E, max_m)
    else:
        masked_m, row = mxg.moe_dispatch(t["ids"], E, max_m)
        a, a_sf = mxg.moe_quantize_gather_nvfp4(t["x"], s["g_x"], t["ids"], row, E, max_m)
    alpha = torch.full((E,), np.float32(s["g_x"]) * np.float32(s["g_w"]), dtype=torch.float32, device=DEV)
    out = sentinel_bf16((E, max_m, N), DEV)
    mxg.mx_grouped_gemm_masked(a, a_sf, t["w13"], t["w13_sf"], alpha, masked_m, out)
    torch.cuda.synchronize()
    ids = np_(t["ids"])
    mm_o, row_o = oracle.dispatch(ids, E, max_m)
    assert np.array_equal(np_(masked_m), mm_o) and np.array_equal(np_(row), row_o)
    xq, xsf = oracle.quantize_nvfp4(np_(t["x"].float()), s["g_x"])
    a_h, asf_h = np_(a), np_(a_sf)
    for tt in range(T):
        for j in range(8):
            e, r = ids[tt, j], row_o[tt, j]
            assert np.array_equal(a_h[e, r], xq[tt]) and np.array_equal(asf_h[e, r], xsf[tt])
    bits = bf16_tensor_bits(out)
    active = np.nonzero(mm_o)[0]
    for e in active:
        m = int(mm_o[e])
        assert (bits[e, m:] == SENT_BF16).all()
        y, S = oracle.gemm_nvfp4_rows(a_h[e], asf_h[e], np.arange(m), np_(t["w13"][e]), np_(t["w13_sf"][e]), H,
                                      float(alpha[0].item()))
        assert_within(bf16_from_bits_np(bits[e, :m]), y, S, f"expert {e}")
    idle = np.nonzero(mm_o == 0)[0]
    assert (bits[idle] == SENT_BF16).all()
    log(f"decode GEMM1 ({path}) ok: {len(active)} active experts, sum masked_m={mm_o.sum()}")


HETERO = ((128, 4096, 7168), (1000, 2048, 7168), (4096, 7168, 2048), (37, 4096, 4096))


def _run_hetero(shapes, seed, sf_dtype=None):
    wl = datagen.hetero_gemm_workload(seed, DEV, shapes)
    groups = []
    for q in wl.tensors["groups"]:
        q = dict(q)
        q["out"] = sentinel_bf16((q["M"], q["N"]), DEV)
        groups.append(q)
    mxg = _mxg()
    mxg.mx_grouped_gemm(groups, sf_dtype=mxg.MXG_E4M3 if sf_dtype is None else sf_dtype)
    torch.cuda.synchronize()
    return groups


@pytest.mark.parametrize("pow2", [False, True])
def test_hetero_gemm_full_size_rows(pow2):
    """Every row of the 37- and 128-row groups, and in the others every row on either side of
    each 256-row M-tile boundary plus a seeded sample, all N columns of each.  With pow2 the
    caller declares the (power-of-two) scales as such and the fp4-MFMA path runs."""
    log(f"heterogeneous NVFP4 grouped GEMM (128,4096,7168) (1000,2048,7168) (4096,7168,2048) (37,4096,4096)"
        f"{' with power-of-two scales declared' if pow2 else ''}")
    groups = _run_hetero(HETERO, 1002, _mxg().MXG_E4M3_POW2 if pow2 else None)
    rng = np.random.default_rng(5)
    for gi, q in enumerate(groups):
        M, N, K = q["M"], q["N"], q["K"]
        bits = bf16_tensor_bits(q["out"])
        assert not (bits == SENT_BF16).any(), f"group {gi}: unwritten outputs"
        if M <= 128:
            rows = list(range(M))
        else:
            edges = [r for b in range(256, M, 256) for r in (b - 1, b)]
            rows = sorted(set(edges + rng.choice(M, size=16, replace=False).tolist() + [0, M - 1]))
        y, S = oracle.gemm_nvfp4_rows(np_(q["a"]), np_(q["a_sf"]), rows, np_(q["b"]), np_(q["b_sf"]), K, q["alpha"])
        assert_within(bf16_from_bits_np(bits[rows]), y, S, f"group {gi}")
        log(f"group {gi} ({M},{N},{K}): {len(rows)} rows ok")


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_hetero_gemm_streaming_shapes_and_ldc(out_dtype):
    # every group takes the weight-streaming kernel (N, K multiples of 128): several M
    # tiles with a ragged tail, an empty group, different depths, a padded output stride
    shapes = ((300, 256, 384), (0, 128, 128), (64, 384, 1024), (513, 128, 256))
    log(f"heterogeneous NVFP4 grouped GEMM, streaming shapes {shapes}, {out_dtype}, ldc = N + 68")
    wl = datagen.hetero_gemm_workload(11, DEV, shapes)
    groups = []
    for q in wl.tensors["groups"]:
        q = dict(q)
        q["ldc"] = q["N"] + 68
        mk = sentinel_bf16 if out_dtype == torch.bfloat16 else sentinel_f32
        q["out"] = mk((max(q["M"], 1), q["ldc"]), DEV)
        groups.append(q)
    _mxg().mx_grouped_gemm(groups, out_dtype=out_dtype)
    torch.cuda.synchronize()
    for gi, q in enumerate(groups):
        M, N, K = q["M"], q["N"], q["K"]
        if M == 0:
            continue
        if out_dtype == torch.bfloat16:
            bits = bf16_tensor_bits(q["out"])
            assert (bits[:, N:] == SENT_BF16).all(), f"group {gi}: padding columns written"
            got = bf16_from_bits_np(bits[:, :N])
        else:
            o = np_(q["out"])
            assert (o[:, N:].view(np.uint32) == np.uint32(SENT_F32 & 0xFFFFFFFF)).all(), \
                f"group {gi}: padding columns written"
            got = o[:, :N].astype(np.float64)
        y, S, _ = oracle.gemm_nvfp4_masked(np_(q["a"])[None], np_(q["a_sf"])[None], np_(q["b"])[None],
                                           np_(q["b_sf"])[None], np.array([q["alpha"]], np.float32),
                                           [M], M, N, K)
        assert_within(got, y[0], S[0], f"group {gi}")


@pytest.mark.parametrize("shapes", [
    ((37, 520, 1024), (0, 64, 128), (130, 600, 128), (1, 16, 64)),
    ((256, 256, 256),),
])
def test_hetero_gemm_tails_full(shapes):
    log(f"heterogeneous NVFP4 grouped GEMM tails {shapes}")
    groups = _run_hetero(shapes, 3)
    for gi, q in enumerate(groups):
        if q["M"] == 0:
            continue
        bits = bf16_tensor_bits(q["out"])
        y, S, _ = oracle.gemm_nvfp4_masked(np_(q["a"])[None], np_(q["a_sf"])[None], np_(q["b"])[None],
                                           np_(q["b_sf"])[None], np.array([q["alpha"]], np.float32),
                                           [q["M"]], q["M"], q["N"], q["K"])
        assert_within(bf16_from_bits_np(bits), y[0], S[0], f"group {gi}")


# ----------------------------------------------------------------------------- contiguous layout
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_contiguous_gemm_groups_and_padding(out_dtype):
    """Expert-sorted rows with aligned padding: groups of 0 to 300 rows (several 256-row M
    tiles, tails inside 16-row groups), every valid row against the oracle, the padding
    rows and the rows past the last group left untouched."""
    counts = [0, 1, 130, 256, 300, 17, 64, 129]
    G, N, K, align = len(counts), 384, 512, 16
    start = [0]
    for c in counts:
        start.append(start[-1] + -(-c // align) * align)
    M_total = start[-1] + 32
    log(f"contiguous grouped NVFP4 GEMM G={G} M_total={M_total} N={N} K={K} {out_dtype}")
    gen = datagen.generator(2024, DEV)
    a, a_sf = datagen.nvfp4_uniform(gen, (M_total,), K, DEV)
    b, b_sf = datagen.nvfp4_uniform(gen, (G, N), K, DEV)
    alpha = torch.linspace(0.05, 0.4, G, device=DEV, dtype=torch.float32)
    gs = torch.tensor(start, dtype=torch.int32, device=DEV)
    cnt = torch.tensor(counts, dtype=torch.int32, device=DEV)
    out = (sentinel_bf16 if out_dtype == torch.bfloat16 else sentinel_f32)((M_total, N), DEV)
    _mxg().mx_grouped_gemm_contiguous(a, a_sf, b, b_sf, alpha, gs, cnt, out)
    torch.cuda.synchronize()
    if out_dtype == torch.bfloat16:
        bits, sent, kw = bf16_tensor_bits(out), SENT_BF16, {}
        vals = bf16_from_bits_np(bits)
    else:
        bits, sent, kw = np_(out.view(torch.int32)).view(np.uint32), SENT_F32 & 0xFFFFFFFF, dict(ulp=ulp_f32)
        vals = np_(out).astype(np.float64)
    a_h, asf_h, b_h, bsf_h, al = np_(a), np_(a_sf), np_(b), np_(b_sf), np_(alpha)
    valid = np.zeros(M_total, bool)
    for g, c in enumerate(counts):
        r0 = start[g]
        valid[r0:r0 + c] = True
        for m in range(c):
            y, S = oracle.nvfp4_row_dot(a_h, asf_h, r0 + m, b_h[g], bsf_h[g], K, float(al[g]))
            assert_within(vals[r0 + m], y, S, f"contiguous group {g} row {m}", **kw)
    assert (bits[~valid] == sent).all(), "padding or trailing rows were written"


@pytest.mark.parametrize("T,E,align", [(37, 16, 8), (4096, 256, 128)])
def test_dispatch_contiguous_matches_oracle(T, E, align):
    log(f"contiguous dispatch T={T} E={E} align={align}")
    gen = datagen.generator(3300 + T, DEV)
    ids = datagen.distinct_topk_ids(gen, T, E, 8, DEV)
    gs, cnt, row = _mxg().moe_dispatch_contiguous(ids, E, align)
    torch.cuda.synchronize()
    s_o, c_o, r_o = oracle.dispatch_contiguous(np_(ids), E, align)
    assert np.array_equal(np_(cnt), c_o) and np.array_equal(np_(gs), s_o) and np.array_equal(np_(row), r_o)


# ----------------------------------------------------------------------------- power-of-two scales
def _pow2_groups(shapes, seed, out_dtype, ldc_pad=0, extreme=False):
    gen = datagen.generator(seed, DEV)
    groups = []
    for gi, (M, N, K) in enumerate(shapes):
        a, a_sf = datagen.nvfp4_uniform(gen, (M,), K, DEV)
        b, b_sf = datagen.nvfp4_uniform(gen, (N,), K, DEV)
        if extreme:
            # every power-of-two e4m3 scale: subnormal 2^-9, 2^-8, 2^-7 and 2^-6 .. 2^8
            codes = torch.tensor([0x01, 0x02, 0x04] + [(u + 7) << 3 for u in range(-6, 9)], dtype=torch.uint8,
                                 device=DEV)
            a_sf = codes[torch.randint(0, len(codes), tuple(a_sf.shape), generator=gen, device=DEV)]
            b_sf = codes[torch.randint(0, len(codes), tuple(b_sf.shape), generator=gen, device=DEV)]
        ldc = N + ldc_pad
        mk = sentinel_bf16 if out_dtype == torch.bfloat16 else sentinel_f32
        groups.append(dict(M=M, N=N, K=K, ldc=ldc, a=a, a_sf=a_sf, b=b, b_sf=b_sf, alpha=0.125 * (gi + 1),
                           out=mk((max(M, 1), ldc), DEV)))
    return groups


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("case", ["tails", "extreme_scales", "many_groups", "fallback_ldc"])
def test_hetero_gemm_pow2_against_oracle(out_dtype, case):
    """The fp4-MFMA path (scales declared powers of two) against the oracle on every output:
    M tails inside and past the first 128 rows of a tile, an empty group, K from one step up,
    padded output rows, every power-of-two scale including the e4m3 subnormals, and more
    groups than one item each."""
    mxg = _mxg()
    if case == "tails":
        shapes, pad, extreme = ((300, 256, 384), (0, 128, 128), (37, 384, 1024), (513, 128, 256), (128, 128, 128),
                                (129, 640, 5120)), 72, False
    elif case == "extreme_scales":
        shapes, pad, extreme = ((200, 256, 512), (16, 128, 896)), 0, True
    elif case == "many_groups":
        shapes, pad, extreme = tuple((17 * g + 1, 128 * (1 + g % 3), 128 * (1 + g % 5)) for g in range(12)), 8, False
    else:  # output rows not 16-byte aligned: the general kernels run, with the same results
        shapes, pad, extreme = ((300, 256, 384), (37, 128, 256)), 2, False
    log(f"power-of-two scales on the fp4 MFMA: {case} {shapes} {out_dtype}")
    groups = _pow2_groups(shapes, 4242 + len(case), out_dtype, pad, extreme)
    mxg.mx_grouped_gemm(groups, out_dtype=out_dtype, sf_dtype=mxg.MXG_E4M3_POW2)
    torch.cuda.synchronize()
    for gi, q in enumerate(groups):
        M, N, K = q["M"], q["N"], q["K"]
        if M == 0:
            continue
        if out_dtype == torch.bfloat16:
            bits = bf16_tensor_bits(q["out"])
            assert (bits[:, N:] == SENT_BF16).all(), f"group {gi}: padding columns written"
            got, kw = bf16_from_bits_np(bits[:, :N]), {}
        else:
            o = np_(q["out"])
            assert (o[:, N:].view(np.uint32) == np.uint32(SENT_F32 & 0xFFFFFFFF)).all(), f"group {gi}: padding written"
            got, kw = o[:, :N].astype(np.float64), dict(ulp=ulp_f32)
        y, S = oracle.gemm_nvfp4_rows(np_(q["a"]), np_(q["a_sf"]), np.arange(M), np_(q["b"]), np_(q["b_sf"]), K,
                                      q["alpha"])
        assert_within(got, y, S, f"pow2 {case} group {gi} ({M},{N},{K})", **kw)


def test_hetero_gemm_exact_grid_independent():
    """The exact heterogeneous path (longest-first item schedule over the resident grid)
    gives the same bits whatever the grid (cu_limit), and matches the oracle."""
    mxg = _mxg()
    shapes = ((300, 256, 384), (1000, 512, 1024), (64, 768, 256), (37, 384, 2048))
    outs = []
    for cu in (0, 7, 64):
        wl = datagen.hetero_gemm_workload(78, DEV, shapes)
        groups = []
        for q in wl.tensors["groups"]:
            q = dict(q)
            q["out"] = torch.empty((q["M"], q["N"]), dtype=torch.float32, device=DEV)
            groups.append(q)
        mxg.mx_grouped_gemm(groups, out_dtype=torch.float32, cu_limit=cu)
        torch.cuda.synchronize()
        outs.append([np_(q["out"]).view(np.uint32) for q in groups])
    for o in outs[1:]:
        assert all(np.array_equal(x, y) for x, y in zip(outs[0], o))
    for gi, q in enumerate(groups):
        M, N, K = q["M"], q["N"], q["K"]
        y, S = oracle.gemm_nvfp4_rows(np_(q["a"]), np_(q["a_sf"]), np.arange(M), np_(q["b"]), np_(q["b_sf"]), K,
                                      q["alpha"])
        assert_within(np_(q["out"]).astype(np.float64), y, S, f"exact group {gi} ({M},{N},{K})", ulp=ulp_f32)


def test_hetero_gemm_pow2_grid_independent():
    """The fp4-MFMA path gives the same bits whatever the grid (cu_limit) and schedule."""
    mxg = _mxg()
    shapes = ((300, 256, 384), (1000, 512, 1024), (64, 768, 256))
    outs = []
    for cu in (0, 7, 64):
        groups = _pow2_groups(shapes, 77, torch.float32)
        mxg.mx_grouped_gemm(groups, out_dtype=torch.float32, sf_dtype=mxg.MXG_E4M3_POW2, cu_limit=cu)
        torch.cuda.synchronize()
        outs.append([np_(q["out"]).view(np.uint32) for q in groups])
    for o in outs[1:]:
        assert all(np.array_equal(x, y) for x, y in zip(outs[0], o))
