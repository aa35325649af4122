"""CPU checks of bench.py's host logic: a committed HBM-traffic summary is reported only while the
kernel source it was taken on is the current one (a changed kernel reports null, never a stale
figure), other sizes get no traffic figure, and a multi-GPU request is refused."""

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


def _current(fname, src):
    return json.load(open(os.path.join(bench.PROFILES, fname))).get("kernel_source_sha256") == \
        bench.kernel_source_sha(src)


@pytest.mark.parametrize("workload", sorted(bench.TRAFFIC))
def test_decode_traffic_only_from_current_kernel_sources(workload):
    fname, src = bench.TRAFFIC[workload]
    want = _recorded(fname) if _current(fname, src) else None
    assert bench.traffic_entry(_args(workload=workload)) == want


def test_fp8_and_prefill_traffic_only_from_current_kernel_sources():
    fname, src = bench.TRAFFIC_FP8["lite_b64"]
    assert bench.traffic_entry(_args(cache="fp8")) == (_recorded(fname) if _current(fname, src) else None)
    fname, src = bench.TRAFFIC_PF
    assert bench.prefill_traffic(_args()) == (_recorded(fname) if _current(fname, src) else None)


def test_stale_summary_reports_null(tmp_path, monkeypatch):
    """A summary whose recorded source hash is not the current one is never reported."""
    fname, src = bench.TRAFFIC["lite_b64"]
    rec = json.load(open(os.path.join(bench.PROFILES, fname)))
    rec["kernel_source_sha256"] = "0" * 64
    (tmp_path / fname).write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.traffic_entry(_args()) is None


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
