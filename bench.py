"""Benchmark of the block-scaled grouped-GEMM / MoE hot path on one MI355X.

Headline workload (one "step" = the whole decode GEMM1 path): 8 tokens routed top-8
to 256 experts (ids from the seed) -> dispatch (masked_m, rows) -> NVFP4 quantization
of the bf16 activations into the masked layout -> masked grouped NVFP4 GEMM1 against
W13 [256, 4096, 7168] with bf16 output.  Inputs are resident in HBM before timing, and the
timed steps follow about 25 ms of untimed back-to-back steps (the loaded steady state).

Prints ONE JSON line with the metric, a roofline object for the dominant kernel
(algorithmic bytes / its HIP-event-timed average duration), cold-cache samples, the
captured-graph replay time of the decode workloads and the oracle's CPU baseline on a
bounded sample.  The default run adds the other four configurations under "workloads"
(the masked GEMM of 4 groups, the heterogeneous GEMM with general and with power-of-two
scales, the FP8 layer at T=4096 and the NVFP4 layer at T=64 and T=8192), each with its roofline against HBM and the MFMA peaks,
tokens/s for the layers and an oracle baseline (token subsets for the prefill layers).
--all adds the rows beyond the configurations (full-precision FP8 intermediate,
interleaved W13, W4A16 GEMV, contiguous layout); --workload X makes X the main line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import datagen  # noqa: E402
import fp8_grouped_gemm_nvfp4_amd as mxg  # noqa: E402

HBM_PEAK_GBS = 8000.0
PEAK_TFLOPS = {"fp16": 2500.0, "bf16": 2500.0, "fp8": 5000.0, "fp4": 10100.0}
NVFP4_ROW_BYTES = lambda K: K // 2 + K // 16  # codes + e4m3 scales per row  # noqa: E731


# HBM traffic of the dominant kernel, measured with rocprofv3 FETCH_SIZE / WRITE_SIZE
# counters (scaled by the same counters on a plain copy of known size) and recorded
# with a hash of the kernel's sources: a record taken from other sources is ignored.
TRAFFIC_RECORDS = {
    "decode_gemm1": ("profiles/decode_gemm1_skinny_hbm_traffic.md",
                     ["fp8_grouped_gemm_nvfp4_amd/csrc/gemm_nvfp4_skinny.hip",
                      "fp8_grouped_gemm_nvfp4_amd/csrc/device_common.h",
                      "fp8_grouped_gemm_nvfp4_amd/csrc/kernels.h"]),
}


def kernel_source_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic(workload):
    """Bytes per launch from the committed counter record, or None when there is no
    record or the kernel's sources changed since it was taken."""
    if workload not in TRAFFIC_RECORDS:
        return None
    path, files = TRAFFIC_RECORDS[workload]
    try:
        text = open(os.path.join(ROOT, path)).read()
    except OSError:
        return None
    m_b = re.search(r"^traffic_bytes_per_launch:\s*(\d+)", text, re.M)
    m_h = re.search(r"^source_sha256:\s*([0-9a-f]{64})", text, re.M)
    if not (m_b and m_h) or m_h.group(1) != kernel_source_hash(files):
        return None
    return int(m_b.group(1))


def copy_calibration(dev, nbytes=1 << 30, reps=3):
    """A plain device copy of known size (nbytes read, nbytes written per launch) whose
    FETCH_SIZE / WRITE_SIZE counters calibrate the counters of the other kernels."""
    src = torch.empty((nbytes,), dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()


def summarize_counters(fetch_csv, write_csv, workload="decode_gemm1", kernel_substr="k_gemm_nvfp4_skinny"):
    """Markdown traffic record from two rocprofv3 --pmc counter_collection.csv files
    (FETCH_SIZE, WRITE_SIZE; KiB per dispatch) of a --copy-calibration run: the
    dominant kernel's counters averaged over its dispatches and scaled by the ratio of
    the known size of the 1 GiB copy to what the same counter reads for it."""
    import csv
    known_kib = (1 << 30) / 1024.0

    def per_kernel(path, counter):
        vals, copy = [], []
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            v = float(r["Counter_Value"])
            if kernel_substr in r["Kernel_Name"]:
                vals.append(v)
            elif "copyBuffer" in r["Kernel_Name"] and v >= 0.25 * known_kib:
                copy.append(v)
        if not vals or not copy:
            raise SystemExit(f"{path}: no {counter} rows for the kernel or for the 1 GiB copy")
        return float(np.mean(vals)), len(vals), float(np.mean(copy))

    f_k, n_f, f_c = per_kernel(fetch_csv, "FETCH_SIZE")
    w_k, n_w, w_c = per_kernel(write_csv, "WRITE_SIZE")
    f_scale, w_scale = known_kib / f_c, known_kib / w_c
    traffic = int(round((f_k * f_scale + w_k * w_scale) * 1024))
    path, files = TRAFFIC_RECORDS[workload]
    lines = [
        f"# HBM traffic of {kernel_substr} ({workload})",
        "",
        "| counter | kernel mean (KiB/dispatch) | dispatches | 1 GiB copy reads (KiB) | scale | scaled bytes |",
        "|---|---|---|---|---|---|",
        f"| FETCH_SIZE | {f_k:.1f} | {n_f} | {f_c:.1f} | {f_scale:.4f} | {int(f_k * f_scale * 1024)} |",
        f"| WRITE_SIZE | {w_k:.1f} | {n_w} | {w_c:.1f} | {w_scale:.4f} | {int(w_k * w_scale * 1024)} |",
        "",
        f"traffic_bytes_per_launch: {traffic}",
        f"source_sha256: {kernel_source_hash(files)}",
        "",
        "sources hashed: " + ", ".join(files),
    ]
    return "\n".join(lines)


# Sources of the MFMA kernels whose counters the MFMA record summarizes.
MFMA_KERNEL_SOURCES = ["fp8_grouped_gemm_nvfp4_amd/csrc/gemm_nvfp4_stream.hip",
                       "fp8_grouped_gemm_nvfp4_amd/csrc/gemm_nvfp4_skinny.hip",
                       "fp8_grouped_gemm_nvfp4_amd/csrc/gemm_nvfp4_mx.hip",
                       "fp8_grouped_gemm_nvfp4_amd/csrc/gemm_fp8.hip",
                       "fp8_grouped_gemm_nvfp4_amd/csrc/stream_common.h",
                       "fp8_grouped_gemm_nvfp4_amd/csrc/device_common.h",
                       "fp8_grouped_gemm_nvfp4_amd/csrc/kernels.h"]
MFMA_KERNELS = {  # kernel name substring -> (MFMA dtype, the instruction's peak), for the record
    "k_gemm_nvfp4_stream": ("fp16", "v_mfma_f32_16x16x32_f16"),
    "k_gemm_nvfp4_skinny": ("fp16", "v_mfma_f32_16x16x32_f16"),
    "k_gemm_nvfp4_mx": ("fp4", "v_mfma_scale_f32_16x16x128_f8f6f4, e2m1 operands"),
    "k_gemm_fp8_swiglu": ("fp8", "v_mfma_scale_f32_16x16x128_f8f6f4, e4m3 operands"),
    "k_gemm_bf16_fp8w": ("bf16", "v_mfma_f32_16x16x32_bf16"),
}


def summarize_mfma_counters(pmc_csv, fetch_csv, write_csv, cus=256, simds_per_cu=4, xcds=8):
    """Markdown record of the MFMA kernels in a rocprofv3 --pmc run (SQ_BUSY_CYCLES,
    SQ_VALU_MFMA_BUSY_CYCLES, SQ_INSTS_VALU, SQ_INSTS_LDS, SQ_LDS_BANK_CONFLICT,
    SQ_INSTS_MFMA, SQ_WAVES, GRBM_GUI_ACTIVE) and two --copy-calibration passes
    (FETCH_SIZE, WRITE_SIZE), averaged per dispatch.  MFMA utilization = MFMA busy cycles
    (summed over SIMDs) over the SIMD cycles of the dispatch (GRBM_GUI_ACTIVE per XCD x
    SIMDs); each busy cycle runs at the peak of the instruction's dtype, so the fraction of
    another dtype's peak scales by the ratio of the peaks."""
    import csv
    from collections import defaultdict

    def per_kernel(path):
        # one row per kernel instantiation (template arguments kept, "void mxg::" dropped)
        out = defaultdict(lambda: defaultdict(list))
        for r in csv.DictReader(open(path)):
            name = r["Kernel_Name"]
            if "copyBuffer" in name:
                key = "copy"
            elif any(k in name for k in MFMA_KERNELS):
                key = name.split("(")[0].replace("void ", "").replace("mxg::", "")
            else:
                continue
            out[key][r["Counter_Name"]].append(float(r["Counter_Value"]))
        return out

    pmc, fet, wri = per_kernel(pmc_csv), per_kernel(fetch_csv), per_kernel(write_csv)
    known_kib = (1 << 30) / 1024.0
    f_scale = known_kib / max(x for x in fet["copy"]["FETCH_SIZE"] if x >= 0.25 * known_kib)
    w_scale = known_kib / max(x for x in wri["copy"]["WRITE_SIZE"] if x >= 0.25 * known_kib)
    lines = ["| kernel | dispatches | MFMA dtype | MFMA instr / dispatch | busy cycles / MFMA | MFMA busy | "
             "of fp16 / fp8 / fp4 peak | VALU instr / wave | LDS instr / wave | LDS bank-conflict cycles / busy | "
             "HBM read MB | HBM write MB |",
             "|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for k in sorted(x for x in pmc if x != "copy"):
        dt, instr = next(v for n, v in MFMA_KERNELS.items() if n in k)
        c = {n: float(np.mean(v)) for n, v in pmc[k].items()}
        simd_cycles = c["GRBM_GUI_ACTIVE"] / xcds * cus * simds_per_cu
        util = c["SQ_VALU_MFMA_BUSY_CYCLES"] / simd_cycles
        rate = util * PEAK_TFLOPS[dt]
        fr = "/".join(f"{rate / PEAK_TFLOPS[p]:.1%}" for p in ("fp16", "fp8", "fp4"))
        rd = float(np.mean(fet[k]["FETCH_SIZE"])) * f_scale * 1024 / 1e6 if k in fet else float("nan")
        wr = float(np.mean(wri[k]["WRITE_SIZE"])) * w_scale * 1024 / 1e6 if k in wri else float("nan")
        per_mfma = c["SQ_VALU_MFMA_BUSY_CYCLES"] / max(c["SQ_INSTS_MFMA"], 1)
        lines.append(f"| `{k}` | {len(pmc[k]['SQ_WAVES'])} | {dt} ({instr}) | {c['SQ_INSTS_MFMA']:.4g} | "
                     f"{per_mfma:.1f} | {util:.1%} | {fr} | "
                     f"{c['SQ_INSTS_VALU'] / c['SQ_WAVES']:.0f} | {c['SQ_INSTS_LDS'] / c['SQ_WAVES']:.0f} | "
                     f"{c['SQ_LDS_BANK_CONFLICT'] / max(c['SQ_BUSY_CYCLES'], 1):.1%} | {rd:.1f} | {wr:.1f} |")
    lines += ["", f"source_sha256: {kernel_source_hash(MFMA_KERNEL_SOURCES)}",
              "sources hashed: " + ", ".join(MFMA_KERNEL_SOURCES),
              f"counter scales from the 1 GiB copy: FETCH_SIZE x{f_scale:.3f}, WRITE_SIZE x{w_scale:.3f}"]
    return "\n".join(lines)


def _ensure_built():
    if not os.path.exists(mxg.LIB_PATH):
        from fp8_grouped_gemm_nvfp4_amd import _build
        _build.build()
    mxg.lib()


class Timer:
    """HIP events on torch's current stream (the stream the library launches on)."""

    def __init__(self):
        self.pairs = []

    def start(self):
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        self.pairs.append([e, None])

    def stop(self):
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        self.pairs[-1][1] = e

    def mean_ms(self):
        return float(np.mean([a.elapsed_time(b) for a, b in self.pairs])) if self.pairs else float("nan")


_SLEEP_CYCLES_PER_MS = None


def gpu_head_start(ms):
    """Occupy the stream with a spin kernel for about `ms` so that the host queues the
    timed launches before the GPU reaches them: the events then bracket GPU work that
    runs back to back, without the host's per-launch gaps."""
    global _SLEEP_CYCLES_PER_MS
    if _SLEEP_CYCLES_PER_MS is None:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(1000)
        a.record()
        torch.cuda._sleep(2_000_000)
        b.record()
        torch.cuda.synchronize()
        _SLEEP_CYCLES_PER_MS = 2_000_000 / max(a.elapsed_time(b), 1e-3)
    torch.cuda._sleep(int(ms * _SLEEP_CYCLES_PER_MS))


# Cold-cache samples of the main workload: each sample is preceded by a 1 GiB scratch
# pass that evicts the L2s and the 256 MB Infinity Cache, then one step is timed alone.
COLD = {"samples": 0, "result": None}


def cold_samples(step, n, nbytes=1 << 30):
    """n samples of one step each after a scrub, with a GPU head start so that the events
    bracket GPU work only.  "dirty": the scrub writes the buffer (the caches then hold
    dirty lines that the step's reads must evict, as after a memset clear of L2);
    "clean": the scrub only reads it."""
    scrub = torch.empty((nbytes,), dtype=torch.uint8, device="cuda")
    scrub.fill_(1)
    out = {"samples": n, "scrub_bytes": nbytes}
    for kind in ("dirty", "clean"):
        times, ktimes = [], []
        for _ in range(n):
            if kind == "dirty":
                scrub.zero_()
            else:
                scrub.view(torch.int64).max()
            gpu_head_start(1.0)
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            kt = Timer()
            a.record()
            step(kt)
            b.record()
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b))
            ktimes.append(kt.mean_ms())
        t, k = np.array(times), np.array(ktimes)
        out[kind] = {"median_ms": float(np.median(t)), "min_ms": float(t.min()),
                     "p90_ms": float(np.percentile(t, 90)), "kernel_median_ms": float(np.median(k))}
    del scrub
    return out


# The timed steps follow at least this much untimed back-to-back GPU work: the host then
# queues the timed launches ahead of the GPU, and the GPU is in its loaded power state (a
# GPU that idled for a few ms runs the next memory-bound launches measurably slower).
HEAD_MS = 25.0


def head_steps(step):
    """Number of untimed steps that take about HEAD_MS, from a timed warm-up step."""
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    step(None)
    b.record()
    torch.cuda.synchronize()
    return int(min(max(np.ceil(HEAD_MS / max(a.elapsed_time(b), 1e-3)), 2), 2000))


def timed_loop(step, steps, warmup):
    for _ in range(warmup):
        step(None)
    torch.cuda.synchronize()
    n_head = head_steps(step)
    kt = Timer()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for _ in range(n_head):
        step(None)
    t0.record()
    for _ in range(steps):
        step(kt)
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    if COLD["samples"] > 0 and COLD["result"] is None:
        COLD["result"] = cold_samples(step, COLD["samples"])
    return t0.elapsed_time(t1) / steps, kt.mean_ms(), wall


def graph_loop(step, steps):
    """Mean time of one step replayed from a captured HIP graph (the pages' grouped
    benchmarks replay pre-captured graphs): the step is captured once after an eager call
    on the capture stream, then replayed `steps` times back to back between two events."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(None)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(None)
    g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    g.replay()
    b.record()
    torch.cuda.synchronize()
    n_head = int(min(max(np.ceil(HEAD_MS / max(a.elapsed_time(b), 1e-3)), 2), 20000))
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    for _ in range(n_head):
        g.replay()
    t0.record()
    for _ in range(steps):
        g.replay()
    t1.record()
    torch.cuda.synchronize()
    del g
    return t0.elapsed_time(t1) / steps


def binding_roof(byts, flops, mfma_dtype):
    """'hbm' or 'mfma': whichever floor (bytes at the HBM peak, flops at the MFMA peak of
    the dtype the path computes in) is longer."""
    return "mfma" if flops / PEAK_TFLOPS[mfma_dtype] / 1e9 > byts / HBM_PEAK_GBS / 1e6 else "hbm"


def roofline_row(r):
    """Roofline view of one workload.  The floor is the longer of its algorithmic bytes at
    the HBM peak and its FLOPs at the MFMA peak of its operand format (fp4 for NVFP4
    operands, fp8 for the FP8 path): `frac` = floor / measured step time.  `of_peak` gives
    the step's rate against each roof separately, and `implementation` the floor at the
    MFMA dtype the kernels actually compute in (the exact NVFP4 decode feeds the fp16
    MFMA, which caps an MFMA-bound NVFP4 workload at 25% of the fp4 peak)."""
    hbm_ms = r["bytes"] / HBM_PEAK_GBS / 1e6
    fmt = r.get("format_dtype", r.get("mfma_dtype", "fp16"))
    impl = r.get("mfma_dtype", fmt)
    fmt_ms = r["flops"] / PEAK_TFLOPS[fmt] / 1e9
    impl_ms = r.get("impl_mfma_ms", r["flops"] / PEAK_TFLOPS[impl] / 1e9)
    floor = max(hbm_ms, fmt_ms)
    of_peak = {"hbm": hbm_ms / r["ms"]}
    for dt in ("fp4", "fp8", "fp16"):
        of_peak[dt] = r["flops"] / PEAK_TFLOPS[dt] / 1e9 / r["ms"]
    return dict(bound="mfma" if fmt_ms > hbm_ms else "hbm", format_dtype=fmt, floor_ms=floor,
                frac=floor / r["ms"], of_peak=of_peak,
                implementation=dict(mfma_dtype=impl, floor_ms=max(hbm_ms, impl_ms),
                                    frac=max(hbm_ms, impl_ms) / r["ms"]))


# ----------------------------------------------------------------------------- workloads
def bench_decode_gemm1(dev, steps, warmup, seed=1001, cpu=True):
    wl = datagen.decode_gemm1_workload(seed, dev)
    t, s = wl.tensors, wl.scalars
    E, T, H, N, top_k, max_m = 256, s["T"], s["H"], s["N"], s["top_k"], 8
    alpha = torch.full((E,), np.float32(s["g_x"]) * np.float32(s["g_w"]), dtype=torch.float32, device=dev)
    masked_m = torch.empty((E,), dtype=torch.int32, device=dev)
    row = torch.empty((T, top_k), dtype=torch.int32, device=dev)
    a = torch.empty((E, max_m, H // 2), dtype=torch.uint8, device=dev)
    a_sf = torch.empty((E, max_m, H // 16), dtype=torch.uint8, device=dev)
    out = torch.empty((E, max_m, N), dtype=torch.bfloat16, device=dev)

    def step(kt):
        # dispatch and quantize-gather in one launch (the batch has 64 slots)
        mxg.moe_dispatch_quantize_gather_nvfp4(t["x"], s["g_x"], t["ids"], E, max_m, masked_m=masked_m, row=row,
                                               a=a, a_sf=a_sf)
        if kt:
            kt.start()
        mxg.mx_grouped_gemm_masked(a, a_sf, t["w13"], t["w13_sf"], alpha, masked_m, out)
        if kt:
            kt.stop()

    ms, kms, wall = timed_loop(step, steps, warmup)
    graph_ms = graph_loop(step, steps)
    mm = masked_m.cpu().numpy()
    n_act, rows = int((mm > 0).sum()), int(mm.sum())
    w_bytes = n_act * N * NVFP4_ROW_BYTES(H)
    gemm_bytes = w_bytes + rows * NVFP4_ROW_BYTES(H) + rows * N * 2
    step_bytes = gemm_bytes + T * H * 2 + T * top_k * 4 * 2 + E * 4
    flops = 2.0 * rows * N * H
    res = dict(name=wl.name, ms=ms, kernel_ms=kms, wall_s=wall, bytes=step_bytes, kernel_bytes=gemm_bytes,
               flops=flops, gbs=step_bytes / ms / 1e6, kernel_gbs=gemm_bytes / kms / 1e6,
               tflops=flops / ms / 1e9, tokens_per_s=T / ms * 1e3, bound="hbm", graph_ms=graph_ms,
               format_dtype="fp4", mfma_dtype="fp16",
               config=dict(workload=wl.name, experts=E, tokens=T, top_k=top_k, K=H, N=N, max_m=max_m,
                           active_experts=n_act, sum_masked_m=rows))
    if cpu:
        res["cpu_baseline"] = cpu_baseline_decode_gemm1(t, s, step_bytes)
    return res


def power_clock_samples(dev, seconds=3.0, seed=1001):
    """Board power (hwmon power1_input), its cap, and the graphics / memory clocks
    (rocm-smi) while the decode GEMM1 runs back to back, with 1 ms and 5 ms idle gaps
    between launches, and after a dispatch kernel per launch as in the timed step; with
    each launch's duration from HIP events (median over the last three quarters)."""
    import glob
    import subprocess
    import threading
    hw = None
    for d in sorted(glob.glob("/sys/class/drm/card*/device/hwmon/hwmon*")):
        if os.path.exists(os.path.join(d, "power1_input")):
            hw = d
            break

    def read(name):
        try:
            return int(open(os.path.join(hw, name)).read())
        except (OSError, TypeError, ValueError):
            return None

    def clocks():
        try:
            r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True, timeout=5)
            card = next(iter(json.loads(r.stdout).values()))
            pick = lambda key: next((int(re.sub(r"[^0-9]", "", v)) for k, v in card.items() if k.startswith(key)), None)
            return pick("sclk clock speed"), pick("mclk clock speed")
        except Exception:  # no rocm-smi or unexpected output: no clock sample
            return None, None

    wl = datagen.decode_gemm1_workload(seed, dev)
    t, sc = wl.tensors, wl.scalars
    E, T, H, N, top_k, max_m = 256, sc["T"], sc["H"], sc["N"], sc["top_k"], 8
    alpha = torch.full((E,), np.float32(sc["g_x"]) * np.float32(sc["g_w"]), dtype=torch.float32, device=dev)
    masked_m = torch.empty((E,), dtype=torch.int32, device=dev)
    row = torch.empty((T, top_k), dtype=torch.int32, device=dev)
    a = torch.empty((E, max_m, H // 2), dtype=torch.uint8, device=dev)
    a_sf = torch.empty((E, max_m, H // 16), dtype=torch.uint8, device=dev)
    out = torch.empty((E, max_m, N), dtype=torch.bfloat16, device=dev)

    def disp():
        mxg.moe_dispatch_quantize_gather_nvfp4(t["x"], sc["g_x"], t["ids"], E, max_m, masked_m=masked_m, row=row,
                                               a=a, a_sf=a_sf)

    def gemm():
        mxg.mx_grouped_gemm_masked(a, a_sf, t["w13"], t["w13_sf"], alpha, masked_m, out)

    disp()
    for _ in range(20):
        gemm()
    torch.cuda.synchronize()
    samples, phase, stop = [], ["idle"], [False]

    def sampler():
        k = 0
        while not stop[0]:
            sclk = mclk = None
            if k % 25 == 0:
                sclk, mclk = clocks()
            samples.append((phase[0], read("power1_input"), sclk, mclk))
            k += 1
            time.sleep(0.01)

    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    time.sleep(1.0)
    kern = {}
    for name, gap in (("back_to_back", 0.0), ("gap_1ms", 1e-3), ("gap_5ms", 5e-3), ("with_dispatch", -1.0)):
        phase[0] = name
        ev, n, t_end = [], 0, time.perf_counter() + seconds
        while time.perf_counter() < t_end:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            if gap < 0:
                disp()
            e0.record()
            gemm()
            e1.record()
            ev.append((e0, e1))
            n += 1
            if gap > 0:
                torch.cuda.synchronize()
                time.sleep(gap)
            elif n % 200 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        ms = np.array([x.elapsed_time(y) for x, y in ev[len(ev) // 4:]])
        kern[name] = {"launches": n, "kernel_us_median": float(np.median(ms)) * 1e3,
                      "kernel_us_p90": float(np.percentile(ms, 90)) * 1e3}
        phase[0] = "idle"
        time.sleep(1.0)
    stop[0] = True
    th.join()
    rows = []
    for name in ("idle", "back_to_back", "gap_1ms", "gap_5ms", "with_dispatch"):
        ss = [x for x in samples if x[0] == name]
        ss = ss[len(ss) // 3:]
        pw = [x[1] for x in ss if x[1] is not None]
        sclk = [x[2] for x in ss if x[2] is not None]
        mclk = [x[3] for x in ss if x[3] is not None]
        k = kern.get(name, {})
        rows.append(f"| {name} | {np.mean(pw) / 1e6 if pw else float('nan'):.0f} | "
                    f"{np.mean(sclk) if sclk else float('nan'):.0f} | {np.mean(mclk) if mclk else float('nan'):.0f} | "
                    f"{k.get('kernel_us_median', float('nan')):.1f} | {k.get('kernel_us_p90', float('nan')):.1f} | "
                    f"{k.get('launches', 0)} |")
    cap = read("power1_cap")
    return "\n".join([f"power cap: {cap / 1e6 if cap else float('nan'):.0f} W (hwmon {hw})", "",
                      "| phase | board power (W) | sclk (MHz) | mclk (MHz) | GEMM us median | GEMM us p90 | launches |",
                      "|---|---|---|---|---|---|---|", *rows])


def cpu_baseline_decode_gemm1(t, s, step_bytes, min_seconds=10.0):
    """The oracle's whole decode GEMM1 path (dispatch, quantize, every valid output row)
    on the host cores, repeated until about min_seconds have elapsed."""
    import oracle
    E, H, N, max_m = 256, s["H"], s["N"], 8
    ids = t["ids"].cpu().numpy()
    x = t["x"].float().cpu().numpy()
    mm, row = oracle.dispatch(ids, E, max_m)
    active = np.nonzero(mm)[0]
    w13 = {int(e): t["w13"][int(e)].cpu().numpy() for e in active}
    w13sf = {int(e): t["w13_sf"][int(e)].cpu().numpy() for e in active}
    alpha = float(np.float32(s["g_x"]) * np.float32(s["g_w"]))
    reps, t0 = 0, time.perf_counter()
    while True:
        mm, row = oracle.dispatch(ids, E, max_m)
        xq, xsf = oracle.quantize_nvfp4(x, s["g_x"])
        for tt in range(ids.shape[0]):
            for j in range(ids.shape[1]):
                e = int(ids[tt, j])
                oracle.nvfp4_row_dot(xq, xsf, tt, w13[e], w13sf[e], H, alpha)
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    return dict(value=step_bytes * reps / el / 1e9, unit="GB/s", cores=oracle.num_threads(), kind="oracle",
                sample=f"the full decode GEMM1 step (dispatch, quantize, all {int(mm.sum())} valid rows x {N} "
                       f"outputs, K={H}) repeated {reps}x in {el:.1f} s",
                seconds_per_step=el / reps)


def bench_masked_c0(dev, steps, warmup, seed=1000, cpu=False):
    wl = datagen.masked_gemm_workload(seed, dev)
    t = wl.tensors
    out = torch.empty((4, 64, 512), dtype=torch.bfloat16, device=dev)

    def step(kt):
        if kt:
            kt.start()
        mxg.mx_grouped_gemm_masked(t["a"], t["a_sf"], t["b"], t["b_sf"], t["alpha"], t["masked_m"], out)
        if kt:
            kt.stop()

    ms, kms, wall = timed_loop(step, steps, warmup)
    mm = t["masked_m"].cpu().numpy()
    rows, ng = int(mm.sum()), int((mm > 0).sum())
    byts = ng * 512 * NVFP4_ROW_BYTES(1024) + rows * NVFP4_ROW_BYTES(1024) + rows * 512 * 2
    flops = 2.0 * rows * 512 * 1024
    res = dict(name=wl.name, ms=ms, kernel_ms=kms, wall_s=wall, bytes=byts, kernel_bytes=byts, flops=flops,
               gbs=byts / ms / 1e6, kernel_gbs=byts / kms / 1e6, tflops=flops / ms / 1e9, bound="launch",
               format_dtype="fp4", mfma_dtype="fp16", config=dict(workload=wl.name, masked_m=mm.tolist()))
    if cpu:
        import oracle
        h = {k: v.cpu().numpy() for k, v in t.items()}
        reps, t0 = 0, time.perf_counter()
        while reps == 0 or time.perf_counter() - t0 < 2.0:
            oracle.gemm_nvfp4_masked(h["a"], h["a_sf"], h["b"], h["b_sf"], h["alpha"], h["masked_m"], 64, 512, 1024)
            reps += 1
        el = time.perf_counter() - t0
        res["cpu_baseline"] = dict(value=byts * reps / el / 1e9, unit="GB/s", cores=oracle.num_threads(),
                                   kind="oracle", sample=f"the whole masked GEMM ({rows} valid rows) x {reps}")
    return res


def bench_hetero(dev, steps, warmup, seed=1002, cpu=False, pow2=False):
    """Config 2.  With pow2 the caller declares the scales (2^u by construction) powers of
    two, and the groups run on the scaled fp4 MFMA."""
    wl = datagen.hetero_gemm_workload(seed, dev)
    sf = mxg.MXG_E4M3_POW2 if pow2 else mxg.MXG_E4M3
    groups = []
    byts, flops = 0, 0.0
    for q in wl.tensors["groups"]:
        q = dict(q)
        q["out"] = torch.empty((q["M"], q["N"]), dtype=torch.bfloat16, device=dev)
        groups.append(q)
        byts += (q["M"] + q["N"]) * NVFP4_ROW_BYTES(q["K"]) + q["M"] * q["N"] * 2
        flops += 2.0 * q["M"] * q["N"] * q["K"]

    def step(kt):
        if kt:
            kt.start()
        mxg.mx_grouped_gemm(groups, sf_dtype=sf)
        if kt:
            kt.stop()

    ms, kms, wall = timed_loop(step, steps, warmup)
    name = wl.name + ("_pow2" if pow2 else "")
    # the power-of-two path: two fp4 MFMAs per 128-K block, i.e. the fp8 rate
    res = dict(name=name, ms=ms, kernel_ms=kms, wall_s=wall, bytes=byts, kernel_bytes=byts, flops=flops,
               gbs=byts / ms / 1e6, tflops=flops / ms / 1e9, kernel_tflops=flops / kms / 1e9, bound="mfma",
               format_dtype="fp4", mfma_dtype="fp8" if pow2 else "fp16",
               config=dict(workload=name, scales="declared powers of two (fp4 MFMA)" if pow2 else "general e4m3"))
    if cpu:
        import oracle
        host = [{k: (v.cpu().numpy() if torch.is_tensor(v) else v) for k, v in q.items() if k != "out"}
                for q in groups]
        t0 = time.perf_counter()
        for q in host:
            oracle.gemm_nvfp4_rows(q["a"], q["a_sf"], np.arange(q["M"]), q["b"], q["b_sf"], q["K"], q["alpha"])
        el = time.perf_counter() - t0
        res["cpu_baseline"] = dict(value=flops / el / 1e12, unit="TFLOP/s", cores=oracle.num_threads(),
                                   kind="oracle", sample=f"every output of the 4 groups ({flops / 2e9:.1f} GMAC), "
                                   f"once, {el:.1f} s")
    return res


GEMV_SHAPES = ((4096, 4096), (14336, 4096), (4096, 14336), (128256, 4096))  # Llama-3-8B (N, K): q/o, gate/up, down, LM head


def bench_gemv_w4a16(dev, steps, warmup, seed=1005, M=1):
    """NVFP4-weight x bf16-activation decode GEMV at batch M over Llama-3-8B (N, K) shapes,
    each timed on its own; the row reports their total bytes over their total time."""
    per = []
    byts_all, ms_all, kms_all, flops_all = 0, 0.0, 0.0, 0.0
    for i, (N, K) in enumerate(GEMV_SHAPES):
        wl = datagen.gemv_w4a16_workload(seed + i, dev, M=M, N=N, K=K)
        t, g_w = wl.tensors, wl.scalars["g_w"]
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)

        def step(kt):
            if kt:
                kt.start()
            mxg.mx_gemv_nvfp4_w4a16(t["x"], t["w"], t["w_sf"], g_w, out=out)
            if kt:
                kt.stop()

        ms, kms, wall = timed_loop(step, steps, warmup)
        byts = N * NVFP4_ROW_BYTES(K) + M * K * 2 + M * N * 2
        per.append(dict(N=N, K=K, us=round(kms * 1e3, 2), gbs=round(byts / kms / 1e6, 1)))
        byts_all += byts
        ms_all += ms
        kms_all += kms
        flops_all += 2.0 * M * N * K
        del t, out
    return dict(name=f"gemv_w4a16_llama3_8b_m{M}", ms=ms_all, kernel_ms=kms_all, wall_s=0.0, bytes=byts_all,
                kernel_bytes=byts_all, flops=flops_all, gbs=byts_all / ms_all / 1e6,
                kernel_gbs=byts_all / kms_all / 1e6, tflops=flops_all / ms_all / 1e9, bound="hbm",
                format_dtype="fp16", mfma_dtype="fp16",
                config=dict(workload=f"gemv_w4a16_llama3_8b_m{M}", M=M, shapes=per))


def bench_contiguous(dev, steps, warmup, seed=1004, T=8192, align=128):
    """GEMM1 of the T=8192 NVFP4 layer over the contiguous (expert-sorted, 128-row aligned)
    layout: routing and contiguous dispatch, then the grouped GEMM on NVFP4 activation
    rows (synthetic codes) against W13, bf16 output."""
    E, H, I, top_k = 256, 7168, 2048, 8
    wl = datagen.moe_nvfp4_workload(seed, dev, T=T)
    t = wl.tensors
    ids, w = mxg.moe_route_noaux(t["logits"], t["bias"], 8, 4, top_k, 2.5)
    gs, cnt, row = mxg.moe_dispatch_contiguous(ids, E, align)
    mm_full, _ = mxg.moe_dispatch(ids, E, 1 << 20)
    torch.cuda.synchronize()
    M_total = int(gs[-1].item())
    cap = max(16, -(-int(mm_full.max().item()) // 16) * 16)
    gen = datagen.generator(seed + 50, dev)
    a, a_sf = datagen.nvfp4_uniform(gen, (M_total,), H, dev)
    alpha = t["g_w13"] * float(datagen.global_scale_from_amax(t["x"]))
    out = torch.empty((M_total, 2 * I), dtype=torch.bfloat16, device=dev)

    def step(kt):
        if kt:
            kt.start()
        mxg.mx_grouped_gemm_contiguous(a, a_sf, t["w13"], t["w13_sf"], alpha, gs, cnt, out)
        if kt:
            kt.stop()

    ms, kms, wall = timed_loop(step, steps, warmup)
    rows = int(cnt.sum().item())
    byts = E * 2 * I * NVFP4_ROW_BYTES(H) + rows * NVFP4_ROW_BYTES(H) + rows * 2 * I * 2
    flops = 2.0 * rows * 2 * I * H
    return dict(name=f"contiguous_gemm1_nvfp4_t{T}", ms=ms, kernel_ms=kms, wall_s=wall, bytes=byts,
                kernel_bytes=byts, flops=flops, gbs=byts / ms / 1e6, tflops=flops / ms / 1e9,
                kernel_tflops=flops / kms / 1e9, bound="mfma", format_dtype="fp4", mfma_dtype="fp16",
                config=dict(workload=f"contiguous_gemm1_nvfp4_t{T}", tokens=T, rows=rows, contiguous_rows=M_total,
                            masked_rows=E * cap, align=align))


def _moe_setup(dev, t, T, E=256, top_k=8):
    ids, w = mxg.moe_route_noaux(t["logits"], t["bias"], 8, 4, top_k, 2.5)
    mm_full, _ = mxg.moe_dispatch(ids, E, 1 << 20)
    cap = max(16, -(-int(mm_full.max().item()) // 16) * 16)
    masked_m, row = mxg.moe_dispatch(ids, E, cap)
    torch.cuda.synchronize()
    return ids, w, masked_m, row, cap


def cpu_baseline_moe(precision, t, s, ids, w, cap, T, n_sub, seed):
    """The oracle's layer on a seeded subset of n_sub tokens (all tokens when n_sub >= T):
    its routing and dispatch run over every token, the expert path (quantize, GEMM1,
    SwiGLU, intermediate, GEMM2, combine) over the subset, which is exact for those tokens
    because the layer is token-separable.  Weights of the touched experts are copied to the
    host before the clock starts."""
    import oracle
    E, I = 256, 2048
    logits, bias = t["logits"].cpu().numpy(), t["bias"].cpu().numpy()
    t0 = time.perf_counter()
    ids_o, w_o = oracle.route_noaux(logits, bias, 8, 4, 8, 2.5)
    mm_o, row_o = oracle.dispatch(ids_o, E, cap)
    t_route = time.perf_counter() - t0
    toks = np.arange(T) if n_sub >= T else np.sort(np.random.default_rng(seed).choice(T, n_sub, replace=False))
    touched = sorted(set(ids_o[toks].ravel().tolist()))
    if precision == "nvfp4":
        W = {e: (t["w13"][e].cpu().numpy(), t["w13_sf"][e].cpu().numpy(), t["w2"][e].cpu().numpy(),
                 t["w2_sf"][e].cpu().numpy()) for e in touched}
        x = t["x"].float().cpu().numpy()
        g13, g2 = t["g_w13"].cpu().numpy(), t["g_w2"].cpu().numpy()
        t0 = time.perf_counter()
        oracle.moe_layer_nvfp4(x, s["g_x"], ids_o, w_o, cap, W.__getitem__, g13, g2, s["g_h"], I, tokens=toks)
    else:
        W = {e: (t["w13"][e].cpu().numpy(), t["w13_s"][e].cpu().numpy(), t["w2"][e].cpu().numpy(),
                 t["w2_s"][e].cpu().numpy()) for e in touched}
        xq, xs = t["xq"].cpu().numpy(), t["xs"].cpu().numpy()
        t0 = time.perf_counter()
        oracle.moe_layer_fp8(xq, xs, ids_o, w_o, cap, W.__getitem__, I, tokens=toks,
                             full_precision_h=precision == "fp8_f32h")
    el = time.perf_counter() - t0
    return dict(value=len(toks) / (el + t_route * len(toks) / T), unit="tokens/s", cores=oracle.num_threads(),
                kind="oracle",
                sample=f"expert path of {len(toks)} of {T} tokens ({len(touched)} experts) in {el:.1f} s; "
                       f"routing + dispatch of all {T} tokens in {t_route:.2f} s, charged pro rata")


def bench_moe(dev, steps, warmup, precision, T, seed, w13_layout=0, cpu=False):
    E, H, I, top_k = 256, 7168, 2048, 8
    fp8 = precision in ("fp8", "fp8_f32h")
    if fp8:
        wl = datagen.moe_fp8_workload(seed, dev, T=T)
    else:
        wl = datagen.moe_nvfp4_workload(seed, dev, T=T)
    t, s = wl.tensors, wl.scalars
    ids, w, masked_m, row, cap = _moe_setup(dev, t, T)
    y = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    if fp8:
        code = mxg.MXG_MOE_FP8_BLOCK128 if precision == "fp8" else mxg.MXG_MOE_FP8_BLOCK128_F32H
        d = mxg.make_moe_desc(code, T, H, I, E, top_k, cap, t["xq"], t["w13"], t["w13_s"],
                              t["w2"], t["w2_s"], ids, w, masked_m, row, y, x_scale=t["xs"])
    else:
        w13, w13_sf = t["w13"], t["w13_sf"]
        if w13_layout:  # the same weights with gate and up rows interleaved in 16-row blocks
            w13, w13_sf = mxg.moe_interleave_w13(w13), mxg.moe_interleave_w13(w13_sf)
            del t["w13"], t["w13_sf"]
            torch.cuda.synchronize()
        d = mxg.make_moe_desc(mxg.MXG_MOE_NVFP4, T, H, I, E, top_k, cap, t["x"], w13, w13_sf,
                              t["w2"], t["w2_sf"], ids, w, masked_m, row, y, g_x=s["g_x"], g_w13=t["g_w13"],
                              g_w2=t["g_w2"], g_h=s["g_h"], w13_layout=w13_layout)
    ws = torch.empty((mxg.moe_expert_forward_workspace_size(d),), dtype=torch.uint8, device=dev)

    def step(kt):
        mxg.moe_route_noaux(t["logits"], t["bias"], 8, 4, top_k, 2.5, ids=ids, w=w)
        mxg.moe_dispatch(ids, E, cap, masked_m=masked_m, row=row)
        if kt:
            kt.start()
        mxg.moe_expert_forward(d, ws)
        if kt:
            kt.stop()

    ms, kms, wall = timed_loop(step, steps, warmup)
    graph_ms = graph_loop(step, steps) if T <= 64 else None
    mm = masked_m.cpu().numpy()
    n_act, rows = int((mm > 0).sum()), int(mm.sum())
    if fp8:
        wbytes = n_act * (2 * I * H + H * I) + n_act * ((2 * I // 128) * (H // 128) + (H // 128) * (I // 128)) * 4
        xbytes = T * H + T * (H // 128) * 4
    else:
        wbytes = n_act * (2 * I * NVFP4_ROW_BYTES(H) + H * NVFP4_ROW_BYTES(I))
        xbytes = T * H * 2
    byts = wbytes + xbytes + T * E * 4 + T * H * 2
    flops = 2.0 * rows * (2 * I * H + H * I)
    # the FP8 GEMMs run on the fp8 MFMA, the exact NVFP4 decode on the fp16 MFMA (the
    # full-precision-intermediate variant's GEMM2 runs twice on the bf16 MFMA; its
    # algorithmic bytes and FLOPs are the layer's, as for the bf16 intermediate)
    mfma_dtype = "fp8" if fp8 else "fp16"
    g1_flops, g2_flops = 2.0 * rows * 2 * I * H, 2.0 * rows * H * I
    if fp8:  # GEMM1 on the scaled fp8 MFMA, GEMM2 on the bf16 MFMA (twice for the hi/lo planes)
        impl_ms = (g1_flops / PEAK_TFLOPS["fp8"] + g2_flops * (2 if precision == "fp8_f32h" else 1)
                   / PEAK_TFLOPS["bf16"]) / 1e9
    else:
        impl_ms = flops / PEAK_TFLOPS["fp16"] / 1e9
    name = wl.name + ("_f32h" if precision == "fp8_f32h" else "") + ("_w13il16" if w13_layout else "")
    res = dict(name=name, ms=ms, kernel_ms=kms, wall_s=wall, bytes=byts, flops=flops,
               gbs=byts / ms / 1e6, tflops=flops / ms / 1e9, tokens_per_s=T / ms * 1e3,
               bound=binding_roof(byts, flops, mfma_dtype), mfma_dtype=mfma_dtype,
               format_dtype="fp8" if fp8 else "fp4", impl_mfma_ms=impl_ms, graph_ms=graph_ms,
               config=dict(workload=name, tokens=T, active_experts=n_act, max_m=cap))
    if cpu:
        res["cpu_baseline"] = cpu_baseline_moe(precision, t, s, ids, w, cap, T, 64 if T <= 64 else 128, seed + 7)
    return res


WORKLOADS = {
    "decode_gemm1": lambda dev, k, w, cpu: bench_decode_gemm1(dev, k, w, cpu=cpu),
    "masked_c0": lambda dev, k, w, cpu: bench_masked_c0(dev, k, w, cpu=cpu),
    "hetero": lambda dev, k, w, cpu: bench_hetero(dev, k, w, cpu=cpu),
    "hetero_pow2": lambda dev, k, w, cpu: bench_hetero(dev, k, w, cpu=False, pow2=True),
    "moe_fp8": lambda dev, k, w, cpu: bench_moe(dev, k, w, "fp8", 4096, 1003, cpu=cpu),
    "moe_fp8_f32h": lambda dev, k, w, cpu: bench_moe(dev, k, w, "fp8_f32h", 4096, 1003, cpu=cpu),
    "moe_nvfp4_decode": lambda dev, k, w, cpu: bench_moe(dev, k, w, "nvfp4", 64, 1004, cpu=cpu),
    "moe_nvfp4_prefill": lambda dev, k, w, cpu: bench_moe(dev, k, w, "nvfp4", 8192, 1004, cpu=cpu),
    "moe_nvfp4_decode_w13il16": lambda dev, k, w, cpu: bench_moe(dev, k, w, "nvfp4", 64, 1004, 16),
    "moe_nvfp4_prefill_w13il16": lambda dev, k, w, cpu: bench_moe(dev, k, w, "nvfp4", 8192, 1004, 16),
    "gemv_w4a16": lambda dev, k, w, cpu: bench_gemv_w4a16(dev, k, w),
    "contiguous_gemm1": lambda dev, k, w, cpu: bench_contiguous(dev, k, w),
}

# The five configurations of the metric: the headline line is the decode GEMM1 (config 1,
# the largest single-GPU configuration the GEMM half of the metric is quoted on); the
# default run adds the other four as rows of "workloads", with the MoE layers' tokens/s.
CONFIG_ROWS = ["masked_c0", "hetero", "hetero_pow2", "moe_fp8", "moe_nvfp4_decode", "moe_nvfp4_prefill"]
# The rows beyond the configurations (--all).
NEXT_ROWS = ["moe_fp8_f32h", "moe_nvfp4_decode_w13il16", "moe_nvfp4_prefill_w13il16", "gemv_w4a16",
             "contiguous_gemm1"]


def table_row(q):
    row = {k: q[k] for k in ("name", "ms", "kernel_ms", "graph_ms", "gbs", "tflops", "tokens_per_s")
           if q.get(k) is not None}
    if "shapes" in q["config"]:
        row["shapes"] = q["config"]["shapes"]
    row["config"] = q["config"]
    row["roofline"] = roofline_row(q)
    if q.get("cpu_baseline") is not None:
        row["cpu_baseline"] = q["cpu_baseline"]
    return row


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode_gemm1", choices=sorted(WORKLOADS))
    ap.add_argument("--all", action="store_true", help="also time the rows beyond the five configurations")
    ap.add_argument("--no-table", action="store_true", help="time the main workload only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold", type=int, default=10,
                    help="cold-cache samples of the main workload (each after a 1 GiB scrub); 0 = none")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration under rocprofv3 --pmc)")
    ap.add_argument("--power-clock", action="store_true",
                    help="print board power and clock samples around back-to-back and gapped decode GEMM1 launches")
    ap.add_argument("--summarize-mfma", nargs=3, metavar=("PMC_CSV", "FETCH_CSV", "WRITE_CSV"),
                    help="print the MFMA-kernel counter record of three rocprofv3 --pmc runs")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="print the traffic record of the dominant kernel from two rocprofv3 --pmc runs")
    args = ap.parse_args()
    if args.summarize_mfma:
        print(summarize_mfma_counters(*args.summarize_mfma))
        return
    if args.summarize_counters:
        print(summarize_counters(*args.summarize_counters, workload=args.workload))
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: the path runs on a single MI355X with no sharding "
              "or collectives; run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    _ensure_built()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.power_clock:
        print(power_clock_samples(dev))
        return
    COLD["samples"] = max(0, args.cold)
    r = WORKLOADS[args.workload](dev, args.steps, args.warmup, not args.no_cpu_baseline)
    COLD["samples"] = 0

    line = {
        "metric": "masked grouped GEMM GB/s & TFLOP/s (% roofline); MoE layer tokens/s, 1 GPU",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": r["ms"], "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "data": "synthetic", "config": r["config"],
    }
    dt = r.get("mfma_dtype", "fp16")
    if r["bound"] == "mfma":
        # against the MFMA peak of the operand format (fp4 for NVFP4, fp8 for FP8); the
        # peak of the dtype the kernels compute in is reported beside it
        fmt = r.get("format_dtype", dt)
        line.update(value=r["tflops"], unit="TFLOP/s", dtype=f"{dt}-mfma/fp32-acc")
        achieved = r["flops"] / r["kernel_ms"] / 1e9
        line["roofline"] = dict(bound="mfma", achieved=achieved, peak=PEAK_TFLOPS[fmt], unit="TFLOP/s",
                                frac=achieved / PEAK_TFLOPS[fmt], traffic=None, peak_dtype=fmt,
                                implementation_peak=PEAK_TFLOPS[dt], implementation_frac=achieved / PEAK_TFLOPS[dt])
    else:
        line.update(value=r["gbs"], unit="GB/s", dtype=f"{dt}-mfma/fp32-acc")
        kb = r.get("kernel_bytes", r["bytes"])
        achieved = kb / r["kernel_ms"] / 1e6
        line["roofline"] = dict(bound="hbm", achieved=achieved, peak=HBM_PEAK_GBS, unit="GB/s",
                                frac=achieved / HBM_PEAK_GBS, traffic=recorded_traffic(args.workload))
    if "tokens_per_s" in r:
        line["tokens_per_s"] = r["tokens_per_s"]
    line["tflops"] = r["tflops"]
    line["kernel_ms"] = r["kernel_ms"]
    if r.get("graph_ms") is not None:
        line["graph_ms_per_step"] = r["graph_ms"]
    if COLD["result"] is not None:
        line["cold"] = COLD["result"]
    line["cpu_baseline"] = r.get("cpu_baseline")
    line["main_roofline"] = roofline_row(r)
    names = [] if args.no_table else [n for n in CONFIG_ROWS + (NEXT_ROWS if args.all else []) if n != args.workload]
    if names:
        rows = []
        for name in names:
            # each row also gets its cold-cache samples (a scrub before every sample)
            COLD["samples"], COLD["result"] = max(0, args.cold), None
            q = WORKLOADS[name](dev, max(10, args.steps // 5), 3, not args.no_cpu_baseline and name in CONFIG_ROWS)
            COLD["samples"] = 0
            row = table_row(q)
            if COLD["result"] is not None:
                row["cold"] = COLD["result"]
            rows.append(row)
            print(f"[bench] {name}: {q['ms']:.4f} ms/step", file=sys.stderr, flush=True)
            del q
            torch.cuda.empty_cache()
        line["workloads"] = rows
    if args.copy_calibration:
        copy_calibration(dev)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
