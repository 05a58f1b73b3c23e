"""CPU tests of bench.py's host logic: kernel-name shortening, the counter
and MFMA profile summaries it writes from rocprofv3 csv files and reads back
(per kernel instantiation, only while the GEMM sources match the recorded
digest), step statistics, and the refusal of more than one GPU.  No GPU and
no torch import are needed."""
import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

GEMM = ("void fgs::(anonymous namespace)::gemm_block_scaled_kernel<fgs::(anonymous namespace)::Shape<2, 4, 4>, "
        "1, 2, true, 0, 0, false>(fgs::(anonymous namespace)::GemmParams)")
GEMM_SHORT = "gemm_block_scaled_kernel<Shape<2, 4, 4>, 1, 2, true, 0, 0, false>"
QUANT = "void fgs::(anonymous namespace)::quant_e4m3_kernel<1, false, false>(unsigned short const*, long)"
STREAM = "void (anonymous namespace)::stream_read_kernel<8, true>(uint4 const*, long, unsigned int*)"
TORCH_FILL = "void at::native::vectorized_elementwise_kernel<16, at::native::FillFunctor<unsigned char> >(int)"
COPY = "__amd_rocclr_copyBuffer"


def _write_counters(d, rows):
    """rows: (kernel name, dispatch id, counter, value[, start ns, end ns])"""
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "c_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"])
        for r in rows:
            name, disp, counter, value = r[:4]
            start, end = r[4:] if len(r) > 4 else (0, 1000)
            w.writerow([disp, name, counter, value, start, end])


def test_kernel_short_names():
    assert bench._kernel_short(GEMM) == GEMM_SHORT
    assert bench._kernel_short(QUANT) == "quant_e4m3_kernel<1, false, false>"
    # the bench's own streaming kernels live in an anonymous namespace at file scope
    assert bench._kernel_short(STREAM) == "stream_read_kernel<8, true>"
    assert bench._kernel_short(COPY) == COPY


def test_counter_profile_round_trip(tmp_path, monkeypatch):
    fetch, write = str(tmp_path / "f"), str(tmp_path / "w")
    cfetch, cwrite = str(tmp_path / "cf"), str(tmp_path / "cw")
    # two dispatches of the GEMM (FETCH 100 and 300 KiB, WRITE 50 and 70 KiB),
    # one of a quantizer, and kernels that are not the library's
    _write_counters(fetch, [(GEMM, 1, "FETCH_SIZE", 100), (GEMM, 2, "FETCH_SIZE", 300), (QUANT, 3, "FETCH_SIZE", 10),
                            (STREAM, 4, "FETCH_SIZE", 999), (TORCH_FILL, 5, "FETCH_SIZE", 1)])
    _write_counters(write, [(GEMM, 1, "WRITE_SIZE", 50), (GEMM, 2, "WRITE_SIZE", 70), (QUANT, 3, "WRITE_SIZE", 20),
                            (STREAM, 4, "WRITE_SIZE", 999), (TORCH_FILL, 5, "WRITE_SIZE", 1)])
    # the 1 GiB copy: FETCH_SIZE reads half the bytes (factor 2), WRITE_SIZE all of them
    _write_counters(cfetch, [(COPY, 1, "FETCH_SIZE", 524288.0)])
    _write_counters(cwrite, [(COPY, 1, "WRITE_SIZE", 1048576.0)])
    out = str(tmp_path / "counters.md")
    bench.write_counter_profile(fetch, write, cfetch, cwrite, ["rocprofv3 ..."], out=out)
    text = open(out).read()
    assert "stream_read_kernel" not in text and "FillFunctor" not in text
    tr = bench.read_kernel_traffic(GEMM_SHORT, path=out)
    assert tr["dispatches"] == 2
    assert tr["fetch_bytes_per_dispatch"] == 200 * 1024 * 2
    assert tr["write_bytes_per_dispatch"] == 60 * 1024
    assert tr["traffic_bytes_per_dispatch"] == 200 * 1024 * 2 + 60 * 1024
    q = bench.read_kernel_traffic("quant_e4m3_kernel<1, false, false>", path=out)
    assert q["traffic_bytes_per_dispatch"] == 10 * 1024 * 2 + 20 * 1024
    assert bench.read_kernel_traffic("no_such_kernel", path=out) is None
    # the figures stop being reported once the GEMM sources change
    monkeypatch.setattr(bench, "gemm_source_digest", lambda: "0" * 16)
    assert bench.read_kernel_traffic(GEMM_SHORT, path=out) is None


def test_counter_profile_rejects_mismatched_dispatch_counts(tmp_path):
    fetch, write = str(tmp_path / "f"), str(tmp_path / "w")
    cfetch, cwrite = str(tmp_path / "cf"), str(tmp_path / "cw")
    _write_counters(fetch, [(GEMM, 1, "FETCH_SIZE", 100), (GEMM, 2, "FETCH_SIZE", 300)])
    _write_counters(write, [(GEMM, 1, "WRITE_SIZE", 50)])
    _write_counters(cfetch, [(COPY, 1, "FETCH_SIZE", 524288.0)])
    _write_counters(cwrite, [(COPY, 1, "WRITE_SIZE", 1048576.0)])
    with pytest.raises(SystemExit):
        bench.write_counter_profile(fetch, write, cfetch, cwrite, [], out=str(tmp_path / "c.md"))


def test_mfma_profile_round_trip(tmp_path, monkeypatch):
    d = str(tmp_path / "m")
    rows = []
    # two dispatches of 1 ms each; per dispatch 2e6 GUI-active cycles per XCD
    # (counter summed over 8 XCDs): 2.0 GHz; MFMA busy 1e6 of 2e6 cycles on
    # each of 1024 SIMDs: 0.5; 1000 MFMAs, 3000 VALU, 250 LDS instructions
    for disp, t0 in ((1, 0), (2, 5_000_000)):
        t1 = t0 + 1_000_000
        for counter, v in (("GRBM_GUI_ACTIVE", 8 * 2e6), ("SQ_VALU_MFMA_BUSY_CYCLES", 1e6 * 1024),
                           ("SQ_INSTS_MFMA", 500), ("SQ_INSTS_VALU", 1500), ("SQ_BUSY_CU_CYCLES", 1),
                           ("SQ_INSTS_VALU_MFMA_MOPS_F16", 1), ("SQ_INSTS_LDS", 125), ("SQ_LDS_BANK_CONFLICT", 0)):
            rows.append((GEMM, disp, counter, v, t0, t1))
    rows.append((QUANT, 3, "SQ_INSTS_VALU", 7, 0, 10))     # not a GEMM: left out
    _write_counters(d, rows)
    out = str(tmp_path / "mfma.md")
    bench.write_mfma_profile(d, ["rocprofv3 ..."], out=out)
    m = bench.read_kernel_mfma(GEMM_SHORT, path=out)
    assert m["dispatches"] == 2
    assert m["mfma_busy"] == pytest.approx(0.5)
    assert m["clock_ghz"] == pytest.approx(2.0)
    assert m["valu_per_mfma"] == pytest.approx(3.0)
    assert m["lds_per_mfma"] == pytest.approx(0.25)
    assert "quant_e4m3_kernel" not in open(out).read()
    monkeypatch.setattr(bench, "gemm_source_digest", lambda: "0" * 16)
    assert bench.read_kernel_mfma(GEMM_SHORT, path=out) is None


def test_mfma_profile_requires_every_counter(tmp_path):
    d = str(tmp_path / "m")
    _write_counters(d, [(GEMM, 1, "GRBM_GUI_ACTIVE", 8e6, 0, 1000)])
    with pytest.raises(SystemExit):
        bench.write_mfma_profile(d, [], out=str(tmp_path / "mfma.md"))


def test_step_stats():
    st = bench.step_stats([k * 1e-3 for k in range(1, 11)])     # 1 .. 10 ms
    assert st["n"] == 10
    assert st["median"] == pytest.approx(5.5)
    assert st["p10"] == pytest.approx(1.9)      # linear interpolation between order statistics
    assert st["p90"] == pytest.approx(9.1)
    assert st["mean"] == pytest.approx(5.5)


def test_committed_profiles_parse():
    """The committed summaries carry a parseable machine-readable block."""
    for path in (bench.COUNTER_PROFILE, bench.MFMA_PROFILE):
        summary = bench._profile_json(path)
        assert summary and "source_digest" in summary and summary["kernels"], path


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
