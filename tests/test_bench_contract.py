"""bench.py's command-line contract: one JSON line with the documented keys
(checked on a GPU with one timed step and no context or CPU baseline), and
a clear refusal of more than one GPU (CPU)."""
import json
import math
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args, timeout=600):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=timeout)


def test_more_than_one_gpu_is_refused():
    r = run_bench("--gpus", "2", timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.gpu
def test_bench_prints_one_json_line_with_the_contract_keys():
    print("[bench contract] bench.py --steps 1 --warmup 1 --no-context --no-cpu", flush=True)
    r = run_bench("--steps", "1", "--warmup", "1", "--no-context", "--no-cpu")
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, f"expected one line on stdout, got {len(lines)}"
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "kernels", "denoise",
                "device_copy"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 1 and d["warmup"] == 1
    assert d["higher_is_better"] is True and d["scaling"] == "weak" and d["data"] == "synthetic"
    assert d["unit"] == "tokens/s" and d["dtype"] == "bf16"
    assert d["vs_baseline"] is None or isinstance(d["vs_baseline"], (int, float))
    assert d["value"] > 0 and d["ms_per_step"] > 0
    cfg = d["config"]
    assert "workload" in cfg and "model" not in cfg
    # whole-job throughput: the step's tokens over its time
    assert math.isclose(d["value"], cfg["tokens_per_step"] / (d["ms_per_step"] * 1e-3), rel_tol=2e-3)
    rl = d["roofline"]
    assert rl["bound"] in ("hbm", "mfma", "alu") and rl["unit"] in ("GB/s", "TFLOP/s")
    assert rl["peak"] > 0 and 0 < rl["achieved"] <= rl["peak"]
    assert math.isclose(rl["frac"], rl["achieved"] / rl["peak"], rel_tol=1e-3)
    assert rl["traffic"] is None or rl["traffic"] > 0
    assert rl["kernel"] in d["kernels"]
    for kind, k in d["kernels"].items():
        assert k["avg_us"] > 0 and k["calls_per_step"] >= 1 and k["of_copy"] > 0, kind
    assert d["device_copy"]["GBps"] > 0
