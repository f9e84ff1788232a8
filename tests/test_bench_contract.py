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


def test_short_kernel_names():
    bench = _bench_module()
    n = bench._short_kernel_name
    assert n("void kda::prefill_prep_kernel<false, 0, true>(bool _Accum const*, kda::SeqLayout, "
             "int)") == "prefill_prep_kernel<false, 0, true>"
    assert n("kda::(anonymous namespace)::decode_multi_mfma_kernel(__bf16 const*, int)") == \
        "decode_multi_mfma_kernel"
    assert n("void kda::varlen_table_kernel(int const*, int)") == "varlen_table_kernel"
    assert n("_ZN3kda13decode_kernelILi128ELi128EDF16bLb0EEEvPKT1_") == "decode_kernel"


def test_record_traffic_from_counter_csv(tmp_path, monkeypatch):
    # two counter runs of 3 calls, 2 kernels with 2 dispatches per call:
    # bytes per call = sum over kernels of (fetch x scale + write x scale) KiB
    # x 1024 x dispatches per call, stored under the workload's key
    import shutil
    bench = _bench_module()
    os.makedirs(tmp_path / "profiles")
    shutil.copy(os.path.join(ROOT, "profiles", "traffic.json"), tmp_path / "profiles")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "feedfacefeedface")
    hdr = "Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n"
    kp = '"void kda::prefill_prep_kernel<false, 0, true>(int)"'
    ks = '"void kda::prefill_state_kernel<false, 1>(int)"'
    for counter, sub, vals in (("FETCH_SIZE", "f", (100.0, 300.0)), ("WRITE_SIZE", "w", (50.0, 10.0))):
        d = tmp_path / sub
        os.makedirs(d / "x")
        rows = []
        for i in range(6):
            rows.append(f"{2 * i},{kp},{counter},{vals[0] + i % 2}")
            rows.append(f"{2 * i + 1},{ks},{counter},{vals[1]}")
        rows.append(f"99,\"void at::native::copy_kernel(int)\",{counter},1e9")   # not a kda kernel
        (d / "x" / "pmc_counter_collection.csv").write_text(hdr + "\n".join(rows) + "\n")
    rec = bench.record_traffic("long", str(tmp_path / "f"), str(tmp_path / "w"), calls=3)
    scales = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    fs, ws = scales["fetch_scale"], scales["write_scale"]
    assert rec["source_hash"] == "feedfacefeedface"
    assert rec["dispatches_per_call"] == {"prefill_prep_kernel<false, 0, true>": 2.0,
                                          "prefill_state_kernel<false, 1>": 2.0}
    want = ((100.5 * fs + 50.5 * ws) + (300.0 * fs + 10.0 * ws)) * 1024 * 2
    assert abs(rec["bytes_per_launch"] - want) < 1e-6 * want
    saved = json.load(open(tmp_path / "profiles" / "traffic.json"))
    key = next(k for k in saved if k.startswith("prefill|") and "T1048576" in k)
    assert saved[key] == rec


def test_traffic_rate():
    bench = _bench_module()
    # 128 GB moved in 25.6 ms is 5 TB/s, 62.5% of the 8 TB/s peak
    r = bench.traffic_rate(128e9, 25.6e3)
    assert abs(r["traffic_gbps"] - 5000.0) < 1e-6
    assert abs(r["traffic_frac"] - 0.625) < 1e-9
    assert bench.traffic_rate(None, 25.6e3) == {"traffic_gbps": None, "traffic_frac": None}
