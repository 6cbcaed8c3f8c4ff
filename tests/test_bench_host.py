"""Host-side logic of bench.py that needs no GPU: the one-GPU guard, the roofline
arithmetic, and the counter-based traffic record (scaling by a copy of known size, and
the source hash that voids a record taken from other kernel sources)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_binding_roof_and_roofline_row():
    # 8 GB at 8 TB/s = 1 ms; 1 TFLOP at 2.5 PFLOP/s = 0.4 ms: HBM-bound
    assert bench.binding_roof(8e9, 1e12, "fp16") == "hbm"
    # 5 TFLOP at 2.5 PFLOP/s = 2 ms > 1 ms
    assert bench.binding_roof(8e9, 5e12, "fp16") == "mfma"
    # the same 5 TFLOP at the fp8 rate take exactly the 1 ms of the bytes: not above it
    assert bench.binding_roof(8e9, 5e12, "fp8") == "hbm"
    row = bench.roofline_row({"bytes": 8e9, "flops": 1e12, "ms": 2.0, "mfma_dtype": "fp16"})
    assert row["bound"] == "hbm" and row["floor_ms"] == pytest.approx(1.0) and row["frac"] == pytest.approx(0.5)
    row = bench.roofline_row({"bytes": 8e9, "flops": 5e12, "ms": 4.0, "mfma_dtype": "fp16"})
    assert row["bound"] == "mfma" and row["floor_ms"] == pytest.approx(2.0) and row["frac"] == pytest.approx(0.5)
    # NVFP4 operands computed on the fp16 MFMA: the floor is at the fp4 peak, the
    # implementation floor at the fp16 one
    row = bench.roofline_row({"bytes": 8e9, "flops": 40.4e12, "ms": 32.0, "format_dtype": "fp4",
                              "mfma_dtype": "fp16"})
    assert row["bound"] == "mfma" and row["floor_ms"] == pytest.approx(4.0) and row["frac"] == pytest.approx(0.125)
    assert row["implementation"]["floor_ms"] == pytest.approx(16.16) and row["of_peak"]["hbm"] == pytest.approx(1 / 32)
    assert row["of_peak"]["fp8"] == pytest.approx(40.4e12 / 5000e9 / 32.0)


def _csv(path, counter, rows):
    with open(path, "w") as f:
        f.write("Kernel_Name,Counter_Name,Counter_Value\n")
        for name, value in rows:
            f.write(f"\"{name}\",{counter},{value}\n")


def test_summarize_counters_scales_by_the_copy(tmp_path):
    kern = "void mxg::k_gemm_nvfp4_skinny<8, 1, 0, 8, 3, 4>(mxg::MaskedGemmArgs)"
    copy = "__amd_rocclr_copyBuffer"
    fetch, write = tmp_path / "fetch.csv", tmp_path / "write.csv"
    # FETCH_SIZE reads half of the 1 GiB copy (factor 2), WRITE_SIZE all of it (factor 1);
    # a small copy below a quarter of the known size is ignored
    _csv(fetch, "FETCH_SIZE", [(kern, 1000), (kern, 1002), (copy, 524288), (copy, 100), (kern, 998)])
    _csv(write, "WRITE_SIZE", [(kern, 10), (copy, 1048576), (kern, 10), (kern, 10)])
    text = bench.summarize_counters(str(fetch), str(write))
    assert "traffic_bytes_per_launch: 2058240" in text          # (1000 * 2 + 10 * 1) KiB
    files = bench.TRAFFIC_RECORDS["decode_gemm1"][1]
    assert f"source_sha256: {bench.kernel_source_hash(files)}" in text


def test_recorded_traffic_follows_the_source_hash(tmp_path, monkeypatch):
    files = bench.TRAFFIC_RECORDS["decode_gemm1"][1]
    good = tmp_path / "good.md"
    bad = tmp_path / "bad.md"
    good.write_text(f"traffic_bytes_per_launch: 123456\nsource_sha256: {bench.kernel_source_hash(files)}\n")
    bad.write_text("traffic_bytes_per_launch: 123456\nsource_sha256: " + "0" * 64 + "\n")
    monkeypatch.setattr(bench, "TRAFFIC_RECORDS", {"decode_gemm1": (str(good), files)})
    assert bench.recorded_traffic("decode_gemm1") == 123456
    monkeypatch.setattr(bench, "TRAFFIC_RECORDS", {"decode_gemm1": (str(bad), files)})
    assert bench.recorded_traffic("decode_gemm1") is None
    assert bench.recorded_traffic("hetero") is None


def _pmc_csv(path, rows):
    with open(path, "w") as f:
        f.write("Kernel_Name,Counter_Name,Counter_Value\n")
        for name, counter, value in rows:
            f.write(f"\"{name}\",{counter},{value}\n")


def test_summarize_mfma_counters(tmp_path):
    kern = "void mxg::k_gemm_nvfp4_mx<0>(mxg::MxGemmArgs)"
    copy = "__amd_rocclr_copyBuffer"
    # one dispatch: 1000 GRBM cycles summed over 8 XCDs = 125 per XCD; 1024 SIMDs;
    # a quarter of the SIMD cycles MFMA-busy
    busy = 0.25 * 125 * 1024
    pmc = [(kern, "GRBM_GUI_ACTIVE", 1000), (kern, "SQ_VALU_MFMA_BUSY_CYCLES", busy), (kern, "SQ_WAVES", 10),
           (kern, "SQ_INSTS_VALU", 500), (kern, "SQ_INSTS_LDS", 70), (kern, "SQ_LDS_BANK_CONFLICT", 5),
           (kern, "SQ_BUSY_CYCLES", 100), (kern, "SQ_INSTS_MFMA", 1)]
    _pmc_csv(tmp_path / "p.csv", pmc)
    _pmc_csv(tmp_path / "f.csv", [(kern, "FETCH_SIZE", 1000), (copy, "FETCH_SIZE", 524288)])
    _pmc_csv(tmp_path / "w.csv", [(kern, "WRITE_SIZE", 100), (copy, "WRITE_SIZE", 1048576)])
    text = bench.summarize_mfma_counters(str(tmp_path / "p.csv"), str(tmp_path / "f.csv"), str(tmp_path / "w.csv"))
    row = next(l for l in text.splitlines() if "`k_gemm_nvfp4_mx<0>`" in l)
    # 25% of the fp4 peak is 2525 TFLOP/s: 101% of fp16, 50.5% of fp8, 25% of fp4
    assert "| 1 | 32000.0 | 25.0% | 101.0%/50.5%/25.0% | 50 | 7 | 5.0% | 2.0 | 0.1 |" in row
    assert f"source_sha256: {bench.kernel_source_hash(bench.MFMA_KERNEL_SOURCES)}" in text
