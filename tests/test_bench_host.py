"""bench.py's command-line contract on the host: one GPU only, a clear exit
without a GPU, and the fields of the timing summary."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=300, cwd=ROOT)


def test_bench_refuses_more_than_one_gpu():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_bench_exits_cleanly_without_a_gpu():
    import torch
    if torch.cuda.is_available():
        import pytest
        pytest.skip("a GPU is visible")
    r = _run("--steps", "1", "--warmup", "0", "--no-cpu-baseline")
    assert r.returncode == 3
    assert "needs a GPU" in r.stderr
    assert r.stdout == ""


def test_timing_fields_report_the_spread_the_settle_phase_and_the_clock():
    sys.path.insert(0, ROOT)
    import bench
    r = {"ms_per_launch": 0.75, "min_ms": 0.74, "median_ms": 0.745, "max_ms": 0.77, "clock_mhz": 1600.0,
         "tflops": 1466.0, "settle_launches": 200, "settle_ms": 151.0}
    t = bench.timing_fields(r, bench.PEAK_TFLOPS["f16"])
    assert t["settle_launches"] == 200 and t["mean_ms"] == 0.75 and t["clock_mhz"] == 1600.0
    assert abs(t["peak_at_clock"] - 2516.6 * 1600 / 2400) < 0.1
    assert abs(t["frac_at_clock"] - 1466.0 / (2516.6 * 1600 / 2400)) < 1e-3
    r["clock_mhz"] = None
    t = bench.timing_fields(r, bench.PEAK_TFLOPS["f16"])
    assert t["clock_mhz"] is None and "frac_at_clock" not in t
