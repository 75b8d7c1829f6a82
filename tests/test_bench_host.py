"""Host-side pieces of bench.py (CPU only): the clock/power sampler's window
summary on synthetic samples, and the multi-GPU refusal."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def sample(t, clks, power, acc, ppt):
    return (t, {"current_gfxclks": clks, "current_gfxclk": 65535, "current_uclk": 1900,
                "current_socket_power": power,
                "accumulation_counter": acc, "ppt_residency_acc": ppt,
                "socket_thm_residency_acc": 0, "temperature_hotspot": 80})


def test_sampler_window_summary():
    s = bench.GpuMetricsSampler()
    # 8 XCD clocks, one unused slot (65535) ignored
    s.samples = [sample(0.0, [2000] * 8 + [65535], 1000, 0, 0),
                 sample(0.05, [1800] * 8 + [65535], 1100, 50, 25),
                 sample(0.10, [1900] * 8 + [65535], 1200, 100, 100),
                 sample(0.50, [100] * 8, 100, 500, 100)]
    w = s.window(0.0, 0.11)
    assert w["samples"] == 3
    assert w["sclk_mhz_median"] == 1900 and w["sclk_mhz_min"] == 1800
    assert w["mclk_mhz_median"] == 1900 and w["socket_power_w_median"] == 1100
    assert w["ppt_limited_frac"] == 1.0 and w["thermal_limited_frac"] == 0.0
    assert s.window(1.0, 2.0) == {"samples": 0}


def test_sampler_reports_its_error():
    s = bench.GpuMetricsSampler()
    s.error = "RuntimeError: no GPU handle"
    assert s.window(0, 1) == {"error": "RuntimeError: no GPU handle"}


def test_launch_spread_and_blas_info():
    per = [1.0, 2.0, 7.0, 4.0, 5.0, 6.0, 3.0]
    assert bench.launch_spread(per) == {"median_launch_ms": 4.0,
                                        "first5_ms": [1.0, 2.0, 7.0, 4.0, 5.0],
                                        "last5_ms": [7.0, 4.0, 5.0, 6.0, 3.0]}
    assert bench.launch_spread([1.0, 3.0])["median_launch_ms"] == 2.0
    info = bench.blas_info()
    assert isinstance(info, list)


def test_timing_record_takes_the_region_average():
    """The record's average step is the timed region's (no events inside
    it); the per-launch pass after it gives only the spread."""
    per = [2.0, 4.0, 3.0]
    r = bench.timing_record(9.3, 3, 0.01, per, {"settle_ms": 2000.0})
    assert r["avg_launch_ms"] == 3.1
    assert r["spread_pass"]["avg_launch_ms"] == 3.0
    assert r["spread_pass"]["min_launch_ms"] == 2.0 and r["spread_pass"]["max_launch_ms"] == 4.0
    assert r["spread_pass"]["median_launch_ms"] == 3.0
    assert r["settle_ms"] == 2000.0 and r["wall_s"] == 0.01


def test_multi_gpu_request_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
