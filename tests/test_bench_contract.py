"""bench.py's contract on the host: one GPU only, and measured HBM traffic is
reported only for the kernel sources it was measured on."""
import importlib.util
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench_module():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""          # no JSON line


def test_traffic_only_for_matching_sources(monkeypatch):
    bench = _bench_module()
    recs = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    key = next(k for k in recs if "|" in k)     # (other keys hold the counter scales)
    kernel, workload = key.split("|", 1)
    rec = recs[key]
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: rec["source_hash"])
    assert bench.measured_traffic(kernel, workload) == rec["bytes_per_launch"]
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 16)
    assert bench.measured_traffic(kernel, workload) is None
    assert bench.measured_traffic("no-such-kernel", workload) is None
