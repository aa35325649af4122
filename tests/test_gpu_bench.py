"""GPU: bench.py end to end in a short run (a few steps, no CPU baseline), in a child process, and the
JSON line it prints: the fields the benchmark contract names, a finite positive value, and the
roofline and traffic entries (traffic: the committed summary's figure for these default sizes when it
was taken on the current kernel sources, null otherwise)."""

import json
import math
import os
import subprocess
import sys

import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _recorded_if_current(fname, src):
    """The traffic a committed summary records, if it was taken on the current kernel sources; else None
    (bench.py reports null for a stale summary)."""
    sys.path.insert(0, ROOT)
    import bench
    rec = json.load(open(os.path.join(bench.PROFILES, fname)))
    return rec.get("traffic_bytes_per_launch") if rec.get("kernel_source_sha256") == bench.kernel_source_sha(src) \
        else None


def _run(*args):
    print("[case] bench.py", *args, flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                       timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    return json.loads(r.stdout.strip().splitlines()[-1])


def test_bench_decode_step_line():
    d = _run("--steps", "5", "--warmup", "2", "--no-cpu-baseline")
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
              "vs_baseline", "dtype", "data", "config", "roofline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 5 and d["warmup"] == 2 and d["unit"] == "GB/s"
    assert math.isfinite(d["value"]) and d["value"] > 0
    assert d["step_calls"] == "mla_decode_step" and "prep" in d["kernels_us"]
    r = d["roofline"]
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and 0 < r["frac"] < 1
    import bench
    assert r["traffic"] == _recorded_if_current(*bench.TRAFFIC["lite_b64"])


def test_bench_prefill_line():
    d = _run("--mode", "prefill", "--steps", "2", "--warmup", "1", "--no-cpu-baseline")
    assert d["unit"] == "TFLOP/s" and math.isfinite(d["value"]) and d["value"] > 0
    r = d["roofline"]
    assert r["bound"] == "mfma" and 0 < r["frac"] < 1
    import bench
    assert r["traffic"] == _recorded_if_current(*bench.TRAFFIC_PF)
