"""Host-side logic of bench.py (no GPU): the one-GPU guard, the clock
arithmetic and the hash check on committed counter records."""
import json
import os
import subprocess
import sys
import threading

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def test_rate_at_clock():
    # 2500 TFLOP/s at 1200 MHz is the whole peak scaled to that clock
    assert bench.at_clock(2500.0, {"gfxclk_mhz": 1200.0})["frac_at_clock"] == 1.0
    assert bench.at_clock(2250.0, {"gfxclk_mhz": 2400.0})["frac_at_clock"] == 0.45
    # no reading: passed through unchanged
    assert bench.at_clock(2000.0, None) is None
    assert bench.at_clock(2000.0, {"error": "x"}) == {"error": "x"}


def _metrics(samples):
    m = bench.GpuMetrics.__new__(bench.GpuMetrics)
    m.samples, m.error, m.power_cap_w, m._thread, m._stop = samples, None, 1400.0, None, threading.Event()
    return m


def test_clock_window_means_and_readings():
    # (time, MHz, W): the values change once a second, sampled more often
    s = [(0.0, 150, 250), (0.5, 150, 250), (1.0, 2000, 1200), (1.5, 2000, 1200), (2.0, 1800, 1300),
         (2.5, 1800, 1300), (3.0, 2400, 900)]
    w = _metrics(s).window(1.0, 2.5)
    assert w["gfxclk_mhz"] == 1900.0 and w["gfxclk_mhz_min"] == 1800
    assert w["socket_power_w"] == 1250.0 and w["samples"] == 4
    assert w["readings"] == 2 and w["readings_mhz_w"] == [[2000, 1200], [1800, 1300]]
    assert "error" in _metrics(s).window(10.0, 11.0)


def test_counter_records_follow_the_kernel_sources(tmp_path):
    h = bench.kernel_source_hash()
    rec = {"kernel_source_sha256": h, "bytes_per_launch": 123, "clock_mhz": 2000, "mfma_busy_of_active": 0.5,
           "launch_us": 250.0, "tflops": 2250.0, "source": "x"}
    p = tmp_path / "rec.json"
    p.write_text(json.dumps(rec))
    assert bench.measured_traffic(str(p)) == 123
    c = bench.measured_clock(str(p))
    assert c["mhz"] == 2000.0 and c["frac_at_clock"] == round(2250.0 / (5000.0 * 2000 / 2400), 4)
    rec["kernel_source_sha256"] = "0" * 64  # taken on other sources: not reported
    p.write_text(json.dumps(rec))
    assert bench.measured_traffic(str(p)) is None and bench.measured_clock(str(p)) is None
    assert bench.measured_traffic(str(tmp_path / "missing.json")) is None


def test_committed_counter_records_match_the_sources():
    # the records under profiles/ were taken on the kernel sources as they are
    assert bench.measured_traffic() is not None
    assert bench.measured_clock() is not None
    assert bench.measured_traffic(bench.KGEMV_TRAFFIC_FILE, bench.KGEMV_SOURCES) is not None
