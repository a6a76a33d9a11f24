"""bench.py's output contract: one JSON line carrying the throughput, the
roofline of the dominant kernel and the CPU oracle's rate, and a refusal of
more than one GPU (the path has no multi-GPU leg)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args, timeout=300):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=timeout, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = run_bench("--gpus", "2", timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stdout + r.stderr


@pytest.mark.gpu
def test_bench_line():
    print("bench.py --steps 3 --warmup 1 (default workload)", flush=True)
    r = run_bench("--steps", "3", "--warmup", "1")
    assert r.returncode == 0, r.stderr[-3000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout[-3000:]
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline", "cpu_baseline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["higher_is_better"] is True and d["scaling"] in ("weak", "strong")
    assert d["vs_baseline"] is None
    assert d["dtype"] == "f32" and d["data"] == "synthetic"
    assert "workload" in d["config"] and "model" not in d["config"]
    # value: (Gaussian, pixel) pairs inside the truncation per second of a step
    assert d["value"] > 0 and d["ms_per_step"] > 0
    assert abs(d["value"] - d["support_pairs"] / (d["ms_per_step"] * 1e-3)) <= 1e-4 * d["value"]

    assert d["tile_lane_pairs"] == 256 * d["tile_pairs"]
    assert 0 < d["tile_lane_efficiency"] <= 1

    rl = d["roofline"]
    assert rl["bound"] in ("hbm", "mfma", "alu")
    assert rl["unit"] in ("GB/s", "TFLOP/s")
    assert 0 < rl["frac"] <= 1
    assert abs(rl["frac"] - rl["achieved"] / rl["peak"]) < 1e-3
    assert rl["traffic"] is None or rl["traffic"] > 0
    assert rl["kernel"] in d["kernels"]
    assert abs(rl["avg_launch_ms"] - d["kernels"][rl["kernel"]]["avg_ms"]) < 1e-9

    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1
    assert cb["unit"] == d["unit"] and cb["sample"]
    # the oracle's fp64 count of the pairs agrees with the GPU's count up to
    # pairs on the truncation edge
    assert cb["support_pairs_rel_diff"] < 1e-5
