"""The numbers bench.py reports from rocprofv3 output (CPU only): kernel time per
run call from a kernel trace, HBM bytes per call from FETCH_SIZE / WRITE_SIZE
scaled by the plain 1 GiB copy of the same run, MFMA-busy from SQ counters, and
the keying of the stored counter summary on line name and kernel sources."""
import csv
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

DEC = "void pkfa::(anonymous namespace)::decode_kernel<1, 4, 3, false, true>(pkfa::AttnParams)"
UP = "pkfa::(anonymous namespace)::upload_kernel(unsigned int*, unsigned int const*, long)"
COPY = "__amd_rocclr_copyBuffer"


def _write_trace(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for name, start_ns, dur_ns in rows:
            w.writerow({"Kernel_Name": name, "Start_Timestamp": start_ns,
                        "End_Timestamp": start_ns + dur_ns})


def _write_counters(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                          "Counter_Value", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for d, name, counter, value, dur_ns in rows:
            w.writerow({"Dispatch_Id": d, "Kernel_Name": name, "Counter_Name": counter,
                        "Counter_Value": value, "Start_Timestamp": 1000 * d,
                        "End_Timestamp": 1000 * d + dur_ns})


@pytest.fixture
def work(monkeypatch):
    # a line's algorithmic bytes without building its workload
    monkeypatch.setattr(bench, "line_work", lambda line: (1_000_000_000, None))


def test_trace_summary_skips_warmup_and_other_kernels(tmp_path, work):
    rows = [(COPY, 0, 50_000)]
    t = 100_000
    for i, dur in enumerate([300_000, 250_000, 100_000, 110_000, 90_000]):   # 2 warmup launches
        rows.append((UP, t, 4_000))
        rows.append((DEC, t + 5_000, dur))
        t += 1_000_000
    d = tmp_path / "trace"
    d.mkdir()
    _write_trace(d / "run_kernel_trace.csv", rows)
    text = bench.summarize("decode_batch64", str(d), "cmd", warmup=2)
    assert "launches 3" in text and "avg_us 100.00" in text
    assert "run_call_avg_us: 100.00" in text
    # 1 GB in 100 us = 10000 GB/s
    assert "achieved: 10000.0 GB/s = 1.2500 of 8000 GB/s HBM peak" in text


def test_counter_summary_scales_by_the_copy(tmp_path, work):
    # the 1 GiB copy reads 524288 KiB of FETCH_SIZE (x 2.0) and writes 1048576 KiB (x 1.0)
    fetch = [(1, COPY, "FETCH_SIZE", 262144.0, 10), (1, COPY, "FETCH_SIZE", 262144.0, 10)]
    write = [(1, COPY, "WRITE_SIZE", 1048576.0, 10)]
    for dsp in (2, 3, 4):                                 # 1 warmup + 2 counted dispatches
        fetch.append((dsp, DEC, "FETCH_SIZE", 500_000.0, 10))
        write.append((dsp, DEC, "WRITE_SIZE", 10_000.0, 10))
    for name, rows in (("fetch", fetch), ("write", write)):
        d = tmp_path / name
        d.mkdir()
        _write_counters(d / "run_counter_collection.csv", rows)
    text = bench.summarize("decode_batch64", f"{tmp_path / 'fetch'},{tmp_path / 'write'}", "cmd",
                           warmup=1)
    fields = dict(l.split(": ", 1) for l in text.splitlines() if ": " in l and not l.startswith("#"))
    assert float(fields["fetch_bytes_per_call"]) == pytest.approx(500_000 * 2.0 * 1024)
    assert float(fields["write_bytes_per_call"]) == pytest.approx(10_000 * 1.0 * 1024)
    hbm = 500_000 * 2.0 * 1024 + 10_000 * 1024
    assert float(fields["hbm_bytes_per_launch"]) == pytest.approx(hbm)
    assert float(fields["traffic_over_algorithmic"]) == pytest.approx(hbm / 1e9, abs=1e-4)


def test_mfma_busy_fraction(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "line_work", lambda line: (1, 1.0))
    app = "void pkfa::(anonymous namespace)::append_kernel<1, 4>(pkfa::AttnParams)"
    rows = []
    for dsp in (1, 2):
        # 8 XCDs x 1e6 active cycles; 1024 SIMDs x 1e6 x 0.4 busy; 1 ms per dispatch
        rows += [(dsp, app, "GRBM_GUI_ACTIVE", 8e6, 1_000_000),
                 (dsp, app, "SQ_VALU_MFMA_BUSY_CYCLES", 0.4 * 1024e6, 1_000_000),
                 (dsp, app, "SQ_BUSY_CU_CYCLES", 0.9 * 256e6, 1_000_000)]
    d = tmp_path / "sq"
    d.mkdir()
    _write_counters(d / "run_counter_collection.csv", rows)
    text = bench.summarize("append_causal_batch16", str(d), "cmd", warmup=1)
    assert "mfma_busy_frac" in text and text.split("mfma_busy_frac")[1].split(": ")[1].startswith("0.4000")
    assert text.split("active_clock_GHz")[1].split(": ")[1].startswith("1.000")
    assert text.split("cu_busy_frac")[1].split(": ")[1].startswith("0.9000")


def test_stored_traffic_keyed_on_line_and_sources(tmp_path, monkeypatch):
    path = tmp_path / "decode_batch64_hbm_counters.txt"
    monkeypatch.setattr(bench, "counters_file", lambda line: str(path))
    monkeypatch.setattr(bench, "kernel_source_sha256", lambda kind="decode": "abc")
    path.write_text("# summary\nline: decode_batch64\nhbm_bytes_per_launch: 643461512\n"
                    "kernel_source_sha256: abc\n")
    assert bench.stored_traffic("decode_batch64") == 643461512
    assert bench.stored_traffic("decode_batch128") is None         # another workload
    path.write_text("# summary\nline: decode_batch64\nhbm_bytes_per_launch: 643461512\n"
                    "kernel_source_sha256: stale\n")
    assert bench.stored_traffic("decode_batch64") is None          # the kernels changed since
