"""Host-side pieces of bench.py (no GPU): the JSON line's shape, the roofline
arithmetic, the CPU-baseline record, the decode step's byte count, and the
refusal of more than one GPU."""

import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


class _Args:
    steps, warmup = 20, 5


def test_line_has_the_contract_keys():
    t = bench.Timing(0.008, 0.0079, 0.0081, 0.00805, 20)
    out = bench.line("m", 1.0, "GB/s", _Args, t, {"workload": "w"}, bench.roofline_hbm(26157628, t))
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
              "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "timing_us"):
        assert k in out, k
    assert out["n_gpus"] == 1 and out["steps"] == 20 and out["warmup"] == 5
    assert out["config"]["workload"] == "w"
    assert out["timing_us"] == {"median": 8.0, "p10": 7.9, "p90": 8.1, "mean": 8.05}
    r = out["roofline"]
    assert r["bound"] == "hbm" and r["peak"] == 8000.0 and r["unit"] == "GB/s"
    # 26157628 bytes in 8 us: 3269.7 GB/s, 40.9% of 8 TB/s
    assert abs(r["achieved"] - 26157628 / 8e-6 / 1e9) < 0.01
    assert abs(r["frac"] - r["achieved"] / 8000.0) < 1e-4


def test_cpu_baseline_record():
    cb = bench.cpu_baseline_rate(0.1, "GB/s", 0.2, 0.1, "a sample")
    for k in ("value", "unit", "cores", "kind", "sample"):
        assert k in cb
    assert cb["cores"] == len(os.sched_getaffinity(0))
    assert cb["kind"] == "oracle"
    assert bench.host_info()["cores"] == len(os.sched_getaffinity(0))


def test_decode_step_bytes_by_hand():
    # Llama-3-8B: per layer q, o 4096x4096; k, v 1024x4096; gate, up 14336x4096;
    # down 4096x14336; the LM head 128256x4096.  W4, FP16 scales and zeros:
    # codes N K / 2, scales and zeros 2 N K / 32 each, x 2 K, y 2 N.
    def w4(N, K):
        return N * K // 2 + 4 * N * (K // 32) + 2 * K + 2 * N
    layer = 2 * w4(4096, 4096) + 2 * w4(1024, 4096) + 2 * w4(14336, 4096) + w4(4096, 14336)
    total = 32 * layer + w4(128256, 4096)
    assert bench.sweep_bytes_per_token(4, 0.0) == total


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_timing_percentiles():
    t = bench.Timing(1.0, 0.5, 2.0, 1.1, 7)
    assert float(t) == 1.0 and t.p10 == 0.5 and t.p90 == 2.0 and t.steps == 7
    assert np.isclose(t.us()["mean"], 1100.0)
