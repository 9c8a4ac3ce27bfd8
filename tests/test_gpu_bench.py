"""bench.py on the GPU: a short run prints exactly one JSON line that keeps the benchmark line's
contract (fields, units, the roofline and CPU-baseline objects, internal consistency)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.gpu
def test_short_bench_run_prints_one_consistent_line(gpu_lib):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "4", "--warmup", "1",
                        "--extra", "causal_32k", "--cpu-seconds", "0.5", "--no-clock"],
                       capture_output=True, text=True, timeout=170, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-3000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
                "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 4 and d["warmup"] == 1
    assert d["unit"] == "TFLOP/s" and d["dtype"] == "bf16" and d["higher_is_better"] is True
    assert d["vs_baseline"] is None and d["config"]["workload"] == "noncausal_16k"
    # value = algorithmic FLOPs of one ring call over the mean time of one timed call
    flops = 4.0 * 128 * 8 * 1 * (16384 * 16384)  # D * Hq * B * visible pairs (non-causal, S = 16384)
    assert d["value"] == pytest.approx(flops / (d["ms_per_step"] * 1e-3) / 1e12, rel=1e-6)
    roof = d["roofline"]
    assert roof["bound"] == "mfma" and roof["unit"] == "TFLOP/s" and roof["peak"] == 2500.0
    assert roof["frac"] == pytest.approx(roof["achieved"] / roof["peak"], rel=1e-9)
    # the step launches cannot take longer than the calls they belong to
    assert roof["launches"] * roof["avg_launch_ms"] <= d["ms_per_step"] * 1.05
    assert 0 < roof["achieved"] < roof["peak"]
    cpu = d["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["unit"] == "TFLOP/s" and cpu["value"] > 0 and cpu["cores"] >= 1
    assert [e["workload"] for e in d["extra"]] == ["causal_32k"]
    g = d["gemm_reference"]
    assert g is None or (g["tflops"] > 0 and g["operands"] == "normal")
