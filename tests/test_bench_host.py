"""CPU checks of bench.py's host logic: the committed HBM-traffic summaries are tied to the kernel
sources they were taken on (a kernel changed without re-profiling shows up here, not as a silent
null in the benchmark line), other sizes get no traffic figure, and a multi-GPU request is refused."""

import argparse
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _args(**kw):
    base = dict(workload="lite_b64", cache="native", seq_len=0, batch=0, pf_batch=4, pf_len=4096)
    base.update(kw)
    return argparse.Namespace(**base)


def _recorded(fname):
    return json.load(open(os.path.join(bench.PROFILES, fname)))["traffic_bytes_per_launch"]


@pytest.mark.parametrize("workload", sorted(bench.TRAFFIC))
def test_decode_traffic_summaries_match_kernel_sources(workload):
    fname, _ = bench.TRAFFIC[workload]
    assert bench.traffic_entry(_args(workload=workload)) == _recorded(fname), \
        f"{fname} was taken on another source of its kernel: re-profile"


def test_fp8_and_prefill_traffic_summaries_match_kernel_sources():
    fname, _ = bench.TRAFFIC_FP8["lite_b64"]
    assert bench.traffic_entry(_args(cache="fp8")) == _recorded(fname)
    assert bench.prefill_traffic(_args()) == _recorded(bench.TRAFFIC_PF[0])


def test_no_traffic_figure_for_other_sizes():
    assert bench.traffic_entry(_args(batch=32)) is None
    assert bench.traffic_entry(_args(seq_len=1024)) is None
    assert bench.traffic_entry(_args(workload="lite_b1")) is None
    assert bench.prefill_traffic(_args(pf_len=2048)) is None


def test_multi_gpu_request_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "exactly one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]
