#!/usr/bin/env python3
"""KDA prefill / decode throughput on one MI355X.

One JSON line on stdout. The headline (``value``) is prefill tokens/s on the
workload chosen with --workload (default: the 1M-token context, B=1, H=32,
T=1,048,576, d=128, chunk 64, bf16 q/k/v, fp32 state: the largest
single-GPU configuration). A "step" is one full prefill of that batch: one
call of kda_prefill_fwd, i.e. chunk cumsum and decay scaling, intra-chunk
Gram, UT inverse, pseudo-values, outputs and the state carry (for few heads
a chunk-parallel prep launch followed by the state-walk launch; the roofline
covers both, timed together with HIP events on their stream). Inputs are
resident in HBM before timing; when a batch is small enough to stay in the
256 MB last-level cache, each timed step reads its own replica of it.

Also reported in the same line: the other two bf16 prefill configurations
(B=1 H=16 T=4096 as "prefill_4k", B=8 H=32 T=8192 with a carried state as
"batched"), each with its own roofline; the decode workload (B=256, H=32,
d=128, 1024 sequential steps, fp32 state of 537 MB streamed per step) as
"decode", an 8-token draft verified and committed from that state as
"decode_multi", a packed batch of 18 prompts of mixed length (65,536 tokens,
H=32) with state checkpoints every 512 tokens as "varlen", the layer form as
"layer", and the fp64 CPU oracle timed on the host cores over a bounded
sample of the headline workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2516.6  # dense bf16 MFMA (256 CU x 2.4 GHz x 4096 flop/clk)
LLC_BYTES = 256 << 20           # Infinity Cache

# Per-step kernel time is one HIP event pair around the whole timed region,
# divided by the step count: the step's kernels plus the short launch gaps
# between them. A timed event pair around every step would add about 8 us of
# wall time to each 80 us prefill step.


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gated_delta_rule_22_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel sources; otherwise None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(path))[f"{kernel}|{workload}"]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_hash") != kernel_source_hash():
        return None
    return rec.get("bytes_per_launch")


def _short_kernel_name(name: str) -> str:
    """'void kda::prefill_prep_kernel<false, 0, true>(args)' -> 'prefill_prep_kernel<false, 0, true>';
    a mangled name ('_ZN3kda13decode_kernelI...') -> its unqualified name ('decode_kernel')."""
    name = name.strip().replace("(anonymous namespace)::", "")
    if name.startswith("_ZN"):
        parts, i = [], 3
        while i < len(name) and name[i].isdigit():
            j = i
            while name[j].isdigit():
                j += 1
            n = int(name[i:j])
            parts.append(name[j:j + n])
            i = j + n
        return parts[-1] if parts else name
    if name.startswith("void "):
        name = name[5:]
    depth, cut = 0, len(name)
    for i, ch in enumerate(name):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            cut = i
            break
    name = name[:cut]
    return name.split("::")[-1] if "<" not in name else name.replace("kda::", "")


def record_traffic(workload: str, fetch_dir: str, write_dir: str, calls: int) -> dict:
    """Write the HBM bytes per call of one workload into profiles/traffic.json
    from two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE; csv output)
    over `calls` calls of that workload, for the kernels of the kda library
    (the decode kernel alone for `decode`). Each counter is averaged per
    dispatch, scaled by the factor recorded from a plain device copy, and
    summed over the dispatches of one call."""
    import csv
    import glob
    import workloads as W

    def per_kernel(d, counter):
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit(f"no counter_collection.csv under {d}")
        tot, cnt = {}, {}
        for f in files:
            for row in csv.DictReader(open(f)):
                kn = row["Kernel_Name"]
                if row["Counter_Name"] != counter or not ("kda::" in kn or kn.startswith("_ZN3kda")):
                    continue
                k = _short_kernel_name(row["Kernel_Name"])
                if workload == "decode" and not k.startswith("decode_kernel"):
                    continue
                tot[k] = tot.get(k, 0.0) + float(row["Counter_Value"])
                cnt[k] = cnt.get(k, 0) + 1
        return {k: tot[k] / cnt[k] for k in tot}, cnt

    fetch, nf = per_kernel(fetch_dir, "FETCH_SIZE")
    write, nw = per_kernel(write_dir, "WRITE_SIZE")
    path = os.path.join(ROOT, "profiles", "traffic.json")
    rec = json.load(open(path))
    fs, ws = rec["fetch_scale"], rec["write_scale"]
    kernels = sorted(fetch)
    per_call = {k: nf[k] / calls for k in kernels}
    total = sum((fetch[k] * fs + write.get(k, 0.0) * ws) * 1024 * per_call[k] for k in kernels)
    cfg = W.DECODE_CONFIGS["decode"] if workload == "decode" else W.PREFILL_CONFIGS[workload]
    key = ("decode|" if workload == "decode" else "prefill|") + cfg.describe()
    rec[key] = {"source_hash": kernel_source_hash(), "kernels": kernels,
                "dispatches_per_call": per_call, "fetch_kib": fetch, "write_kib": write,
                "bytes_per_launch": total}
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    return rec[key]


def bench_prefill(cfg, steps, warmup):
    import torch
    import gated_delta_rule_22_amd as kda
    import workloads as W
    from workloads import accounting as A

    dev = torch.device("cuda:0")
    # a single long sequence is drawn head by head (per-head seeds), as the
    # parity tests draw it
    x = (W.prefill_inputs_by_head(cfg, device=dev) if cfg.name == "long"
         else W.prefill_inputs(cfg, device=dev))
    per_batch = sum(t.numel() * t.element_size() for t in x.values() if t is not None)
    reps = max(1, min(steps + warmup, math.ceil(2 * LLC_BYTES / per_batch)))
    batches = [x] + [{n: (t.clone() if t is not None else None) for n, t in x.items()}
                     for _ in range(reps - 1)]
    outs = [(torch.empty_like(b["v"]),
             torch.empty((cfg.B, cfg.H, cfg.dk, cfg.dv), dtype=torch.float32, device=dev))
            for b in batches]

    ws_bytes = kda.kda_prefill_workspace_size(cfg.B, cfg.T, cfg.H, cfg.dk, cfg.dv, cfg.dtype,
                                              cfg.chunk)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)

    def step(i):
        b = batches[i % reps]
        o, S = outs[i % reps]
        kda.kda_prefill_fwd(b["q"], b["k"], b["v"], b["log_alpha"], b["beta"], b["S0"],
                            chunk=cfg.chunk, o=o, S_final=S, workspace=ws)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(steps):
        step(warmup + i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = ev0.elapsed_time(ev1) / steps

    tokens = cfg.B * cfg.T
    flops = A.prefill_flops(cfg.B, cfg.T, cfg.H, cfg.dk, cfg.chunk)
    flops_c = A.prefill_flops_conservative(cfg.B, cfg.T, cfg.H, cfg.dk, cfg.chunk)
    nbytes = A.prefill_bytes(cfg.B, cfg.T, cfg.H, cfg.dk, cfg.dv, elt=2,
                             has_s0=cfg.s0_std > 0, writes_state=True)
    t = kern_ms * 1e-3
    del batches, outs, ws, x
    torch.cuda.empty_cache()
    return dict(wall_s=wall, ms_per_step=wall * 1e3 / steps, kernel_ms=kern_ms,
                tokens_per_s=tokens * steps / wall, flops=flops, flops_cons=flops_c,
                bytes=nbytes, gbs=nbytes / t / 1e9, tflops=flops / t / 1e12,
                tflops_cons=flops_c / t / 1e12, replicas=reps, workspace_bytes=ws_bytes)


def bench_decode(cfg, loops=2):
    import torch
    import gated_delta_rule_22_amd as kda
    import workloads as W
    from workloads import accounting as A

    dev = torch.device("cuda:0")
    S0 = W.decode_state(cfg, device=dev)
    S = torch.empty_like(S0)
    steps = [W.decode_step_inputs(cfg, s, device=dev) for s in range(cfg.steps)]
    o = torch.empty((cfg.B, cfg.H, cfg.dv), dtype=cfg.dtype, device=dev)
    stream = torch.cuda.current_stream()

    def run():
        for s in steps:
            kda.kda_decode_step(s["q"], s["k"], s["v"], s["log_alpha"], s["beta"], S, o=o)

    S.copy_(S0)
    run()  # warm-up pass
    best = None
    for _ in range(loops):
        S.copy_(S0)
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        ev0.record(stream)
        run()
        ev1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        kern_ms = ev0.elapsed_time(ev1) / cfg.steps
        if best is None or wall < best[0]:
            best = (wall, kern_ms)
    wall, kern_ms = best
    nbytes = A.decode_step_bytes(cfg.B, cfg.H, cfg.dk, cfg.dv)
    return dict(steps=cfg.steps, wall_s=wall, steps_per_s=cfg.steps / wall,
                tokens_per_s=cfg.B * cfg.steps / wall, kernel_us=kern_ms * 1e3,
                bytes_per_step=nbytes, gbs=nbytes / (kern_ms * 1e-3) / 1e9,
                flops_per_step=A.decode_step_flops(cfg.B, cfg.H, cfg.dk, cfg.dv))


def bench_decode_multi(cfg, T=8, reps=20):
    """An 8-token draft from the decode configuration's state: a verify pass
    (n_commit = 0, the state is only read) and a full commit (n_commit = T)."""
    import torch
    import dataclasses
    import gated_delta_rule_22_amd as kda
    import workloads as W
    from workloads import accounting as A

    dev = torch.device("cuda:0")
    S = W.decode_state(cfg, device=dev)
    x = W.prefill_inputs(dataclasses.replace(W.PREFILL_CONFIGS["prefill"]), B=cfg.B, T=T,
                         H=cfg.H, seed=cfg.seed + 77, device=dev)
    o = torch.empty((cfg.B, T, cfg.H, cfg.dv), dtype=cfg.dtype, device=dev)
    zeros = torch.zeros(cfg.B, dtype=torch.int32, device=dev)
    full = torch.full((cfg.B,), T, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    out = {}
    for name, n in (("verify", zeros), ("commit", full)):
        def call():
            kda.kda_decode_multi(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], S,
                                 n_commit=n, o=o)
        call()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for a, b in ev:
            a.record(stream)
            call()
            b.record(stream)
        torch.cuda.synchronize()
        us = sum(a.elapsed_time(b) for a, b in ev) / reps * 1e3
        nbytes = A.decode_multi_bytes(cfg.B, cfg.H, T, cfg.dk, cfg.dv, commit=name == "commit")
        out[name] = {"us_per_call": us, "tokens_per_s": cfg.B * T / (us * 1e-6),
                     "roofline": {"bound": "hbm", "achieved": nbytes / (us * 1e-6) / 1e9,
                                  "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                  "frac": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                                  "kernel": "decode_multi_mfma_kernel", "algorithmic_bytes": nbytes}}
    out["workload"] = f"kda_decode_multi B{cfg.B} H{cfg.H} dk{cfg.dk} dv{cfg.dv} T{T} bf16"
    return out


def bench_varlen(vc, reps=5):
    """The packed serving-style batch (mixed prompt lengths, one kda_prefill_varlen
    call) with and without state checkpoints."""
    import torch
    import gated_delta_rule_22_amd as kda
    import workloads as W
    from workloads import accounting as A

    dev = torch.device("cuda:0")
    base = W.PREFILL_CONFIGS[vc.base]
    lengths = W.varlen_lengths(vc.total, vc.len_lo, vc.len_hi, vc.seed)
    x = W.varlen_inputs(base, lengths, H=vc.H, seed=vc.seed, device=dev)
    cu = x["cu_seqlens"].to(dev)
    N, T, H = len(lengths), vc.total, vc.H
    o = torch.empty_like(x["v"])
    Sf = torch.empty((N, H, base.dk, base.dv), dtype=torch.float32, device=dev)
    n_ck = sum(n // vc.ckpt_every for n in lengths)
    Sc = torch.empty((max(n_ck, 1), H, base.dk, base.dv), dtype=torch.float32, device=dev)
    ws = torch.empty(kda.kda_prefill_varlen_workspace_size(N, T, H, base.dk, base.dv,
                                                           base.dtype), dtype=torch.uint8,
                     device=dev)
    stream = torch.cuda.current_stream()
    out = {"workload": vc.describe(), "sequences": N, "longest": max(lengths)}
    for name, every in (("ckpt", vc.ckpt_every), ("no_ckpt", 0)):
        def call():
            kda.kda_prefill_varlen(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], cu,
                                   x["S0"], ckpt_every=every, o=o, S_final=Sf,
                                   S_ckpt=Sc if every else None, workspace=ws)
        call()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for a, b in ev:
            a.record(stream)
            call()
            b.record(stream)
        torch.cuda.synchronize()
        us = sum(a.elapsed_time(b) for a, b in ev) / reps * 1e3
        nbytes = A.prefill_bytes(1, T, H, base.dk, base.dv, elt=2, has_s0=True,
                                 writes_state=False) + N * H * 4 * base.dk * base.dv
        if every:
            nbytes += n_ck * H * 4 * base.dk * base.dv
        out[name] = {"us_per_call": us, "tokens_per_s": T / (us * 1e-6), "checkpoints": n_ck if every else 0,
                     "roofline": {"bound": "hbm", "achieved": nbytes / (us * 1e-6) / 1e9,
                                  "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                  "frac": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                                  "algorithmic_bytes": nbytes}}
    return out


def _time_calls(call, reps, stream, before=None):
    """Mean HIP-event time of `call` in us; `before` (untimed) runs ahead of
    each call, e.g. to restore a state the call updates in place."""
    import torch
    if before:
        before()
    call()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for a, b in ev:
        if before:
            before()
        a.record(stream)
        call()
        b.record(stream)
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in ev) / reps * 1e3


def bench_layer(cfg, reps=20):
    """The layer form on the prefill workload: raw q, k normalised in the
    kernel, the bounded gate (bf16 pre-activation) or the per-head scalar gate,
    and the output norm-gate epilogue; and a decode step in the layer form on
    the decode configuration. Timed beside the plain op."""
    import torch
    import gated_delta_rule_22_amd as kda
    import workloads as W

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    x = W.layer_inputs(cfg, device=dev)
    la = (-5.0 * torch.sigmoid(x["g"].float())).contiguous()
    o = torch.empty_like(x["v"])
    Sf = torch.empty((cfg.B, cfg.H, cfg.dk, cfg.dv), dtype=torch.float32, device=dev)
    ws_bytes = kda.kda_prefill_workspace_size(cfg.B, cfg.T, cfg.H, cfg.dk, cfg.dv, cfg.dtype)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    tok_heads = cfg.B * cfg.T * cfg.H
    elt = 2
    out = {"workload": cfg.describe()}
    runs = {
        "plain": (lambda: kda.kda_prefill_fwd(x["q"], x["k"], x["v"], la, x["beta"], x["S0"],
                                              o=o, S_final=Sf, workspace=ws),
                  elt * 4 * cfg.dk + 4 * cfg.dk + 4),
        "bounded_l2_normgate": (lambda: kda.kda_prefill_layer(
            x["q"], x["k"], x["v"], x["g"], x["beta"], x["S0"], gate_mode=kda.KDA_GATE_BOUNDED,
            l2norm=True, z=x["z"], w=x["w"], o=o, S_final=Sf, workspace=ws),
            elt * 6 * cfg.dk + 4),
        "scalar_gate_l2": (lambda: kda.kda_prefill_layer(
            x["q"], x["k"], x["v"], x["a"], x["beta"], x["S0"], gate_mode=kda.KDA_GATE_SCALAR,
            l2norm=True, o=o, S_final=Sf, workspace=ws),
            elt * 4 * cfg.dk + 8),
    }
    for name, (call, per_tok) in runs.items():
        us = _time_calls(call, reps, stream)
        nbytes = tok_heads * per_tok + cfg.B * cfg.H * 4 * cfg.dk * cfg.dv * (
            1 + (cfg.s0_std > 0))
        out[name] = {"us_per_call": us, "tokens_per_s": cfg.B * cfg.T / (us * 1e-6),
                     "algorithmic_bytes": nbytes,
                     "hbm_frac": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS}
    # decode step, layer form (bounded gate, L2, norm-gate fused in the kernel)
    dc = W.DECODE_CONFIGS["decode"]
    import dataclasses
    xd = W.layer_inputs(dataclasses.replace(cfg, dk=dc.dk, dv=dc.dv), B=dc.B, H=dc.H,
                        decode=True, device=dev)
    S = W.decode_state(dc, device=dev)
    od = torch.empty_like(xd["v"])
    # A gate pre-activation shifted down so that the per-step decay is mild
    # (-5 sigmoid(g) of about -0.01): the repeated steps on one state keep it
    # at its scale instead of driving it to zero. The plain step takes the
    # same log-decay and the keys that the layer form normalises in the kernel.
    g = (xd["g"].float() - 6.0).to(xd["g"].dtype)
    lad = (-5.0 * torch.sigmoid(g.float())).contiguous()
    qn = torch.nn.functional.normalize(xd["q"].float(), dim=-1).to(xd["q"].dtype)
    kn = torch.nn.functional.normalize(xd["k"].float(), dim=-1).to(xd["k"].dtype)
    us_plain = _time_calls(lambda: kda.kda_decode_step(qn, kn, xd["v"], lad, xd["beta"], S, o=od),
                           reps, stream)
    us_layer = _time_calls(lambda: kda.kda_decode_layer(
        xd["q"], xd["k"], xd["v"], g, xd["beta"], S, gate_mode=kda.KDA_GATE_BOUNDED,
        l2norm=True, z=xd["z"], w=xd["w"], o=od), reps, stream)
    out["decode"] = {"workload": dc.describe().replace("1024 steps ", ""),
                     "plain_us": us_plain, "bounded_l2_normgate_us": us_layer}
    return out


def traffic_rate(traffic, kernel_us):
    """The measured HBM bytes per launch over the same launch time: how close
    the kernels run to the memory system for the bytes they actually move
    (None when the counters do not match the current sources)."""
    if traffic is None:
        return {"traffic_gbps": None, "traffic_frac": None}
    gbs = traffic / (kernel_us * 1e-6) / 1e9
    return {"traffic_gbps": gbs, "traffic_frac": gbs / HBM_PEAK_GBS}


def prefill_roofline(pre, workload):
    kernels = ("prefill_prep_kernel + prefill_state_kernel" if pre["workspace_bytes"] > 0
               else "prefill_fused_kernel")
    traffic = measured_traffic("prefill", workload)
    return {"bound": "hbm", "achieved": pre["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": pre["gbs"] / HBM_PEAK_GBS, "traffic": traffic,
            **traffic_rate(traffic, pre["kernel_ms"] * 1e3),
            "kernel": kernels, "kernel_us": pre["kernel_ms"] * 1e3,
            "algorithmic_bytes": pre["bytes"]}


def prefill_mfma(pre):
    return {"flops_per_step": pre["flops"], "achieved_tflops": pre["tflops"],
            "peak_tflops": MFMA_BF16_PEAK_TFLOPS, "frac": pre["tflops"] / MFMA_BF16_PEAK_TFLOPS,
            "frac_without_inverse": pre["tflops_cons"] / MFMA_BF16_PEAK_TFLOPS}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline_prefill(cfg, max_heads, max_tokens=1 << 16, min_seconds=10.0):
    """fp64 oracle on the host cores over a bounded sample of the same
    workload: whole heads (one per thread) over the first tokens of the
    sequence (the same per-head draws). Inputs are converted before the clock
    starts."""
    import oracle
    import workloads as W

    heads = min(cfg.H, max_heads)
    T = min(cfg.T, max_tokens)
    xs = [W.prefill_inputs_per_head(cfg, h, T=T) for h in range(heads)]
    f64 = lambda key: np.ascontiguousarray(
        np.concatenate([x[key].double().numpy() for x in xs], axis=2))
    q, k, v, la, beta = (f64(n) for n in ("q", "k", "v", "log_alpha", "beta"))
    S0 = None
    if xs[0]["S0"] is not None:
        S0 = np.ascontiguousarray(np.concatenate([x["S0"].double().numpy() for x in xs], axis=1))
    threads = min(os.cpu_count() or 1, heads)
    # repeat the sample until about min_seconds of CPU time have been spent
    passes, t0 = 0, time.perf_counter()
    while True:
        oracle.prefill_f64(q, k, v, la, beta, S0, nthreads=threads)
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    # token-heads per second over the sample, as tokens/s of the full workload
    tps = passes * heads * T / dt / (cfg.B * cfg.H)
    return dict(value=tps, unit="tokens/s", cores=threads, kind="oracle",
                cpu_model=cpu_model(), host_cpus=os.cpu_count(),
                sample=f"{heads} of {cfg.B * cfg.H} sequence-heads x first {T} of {cfg.T} "
                       f"tokens, fp64 token loop, {passes} passes in {dt:.1f} s on {threads} "
                       f"threads; rate scaled to all {cfg.B * cfg.H} sequence-heads")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="long", choices=["prefill", "batched", "long"])
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the other prefill configurations")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-varlen", action="store_true")
    ap.add_argument("--no-layer", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 5 times (calibrates "
                         "the HBM byte counters against a known traffic)")
    ap.add_argument("--record-traffic", nargs=3, metavar=("WORKLOAD", "FETCH_DIR", "WRITE_DIR"),
                    help="no GPU work: store the HBM bytes per call of WORKLOAD (prefill, "
                         "batched, long or decode) in profiles/traffic.json from the csv "
                         "output of two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE)")
    ap.add_argument("--calls", type=int, default=3,
                    help="calls of the workload in those runs (with --record-traffic)")
    args = ap.parse_args()
    if args.record_traffic:
        wl, fd, wd = args.record_traffic
        print(json.dumps(record_traffic(wl, fd, wd, args.calls)))
        return

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the KDA path here "
              "has no multi-GPU mode.", file=sys.stderr)
        sys.exit(2)

    import torch
    import gated_delta_rule_22_amd as kda
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        # a plain device copy: known HBM traffic for the counter scale factors,
        # and the copy rate as a practical streaming reference
        n = 1 << 30
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(5)]
        for a, b in ev:
            a.record()
            dst.copy_(src)
            b.record()
        torch.cuda.synchronize()
        best_ms = min(a.elapsed_time(b) for a, b in ev)
        print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n, "copies": 5,
                          "best_copy_us": best_ms * 1e3,
                          "copy_read_plus_write_gbs": 2 * n / (best_ms * 1e-3) / 1e9}))
        return
    kda.load_library()
    cfg = W.PREFILL_CONFIGS[args.workload]
    steps = args.steps
    _log(f"[bench] prefill {cfg.describe()}: warmup {args.warmup}, steps {steps}")
    pre = bench_prefill(cfg, steps, args.warmup)
    _log(f"[bench] prefill kernel {pre['kernel_ms'] * 1e3:.1f} us, {pre['gbs']:.0f} GB/s, "
         f"{pre['tflops']:.1f} TFLOP/s")

    workload = cfg.describe()
    result = {
        "metric": "KDA prefill tokens/s + % bf16 MFMA peak; decode steps/s + % HBM BW",
        "value": pre["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": pre["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": workload, "B": cfg.B, "T": cfg.T, "H": cfg.H, "dk": cfg.dk,
                   "dv": cfg.dv, "chunk": cfg.chunk, "state": "fp32",
                   "input_replicas": pre["replicas"], "workspace_bytes": pre["workspace_bytes"]},
        "roofline": prefill_roofline(pre, workload),
        "mfma": prefill_mfma(pre),
    }

    # the other bf16 prefill configurations, each with its own roofline
    for key, name in (("prefill_4k", "prefill"), ("batched", "batched"), ("long", "long")):
        if args.no_extra or name == args.workload:
            continue
        c = W.PREFILL_CONFIGS[name]
        _log(f"[bench] {key}: {c.describe()}")
        ex = bench_prefill(c, 20 if name != "long" else 5, 5 if name != "long" else 2)
        _log(f"[bench] {key} {ex['kernel_ms'] * 1e3:.1f} us, {ex['gbs']:.0f} GB/s")
        result[key] = {"workload": c.describe(), "us_per_call": ex["kernel_ms"] * 1e3,
                       "tokens_per_s": ex["tokens_per_s"],
                       "roofline": prefill_roofline(ex, c.describe()), "mfma": prefill_mfma(ex)}

    if not args.no_decode:
        dc = W.DECODE_CONFIGS["decode"]
        _log(f"[bench] decode {dc.describe()}")
        dec = bench_decode(dc)
        _log(f"[bench] decode {dec['kernel_us']:.1f} us/step, {dec['gbs']:.0f} GB/s")
        dtraffic = measured_traffic("decode", dc.describe())
        result["decode"] = {
            "workload": dc.describe(), "steps_per_s": dec["steps_per_s"],
            "tokens_per_s": dec["tokens_per_s"], "us_per_step": dec["wall_s"] / dec["steps"] * 1e6,
            "roofline": {"bound": "hbm", "achieved": dec["gbs"], "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": dec["gbs"] / HBM_PEAK_GBS,
                         "traffic": dtraffic, **traffic_rate(dtraffic, dec["kernel_us"]),
                         "kernel": "decode_kernel", "kernel_us": dec["kernel_us"],
                         "algorithmic_bytes": dec["bytes_per_step"]},
        }

        _log("[bench] decode_multi (8-token draft: verify, commit)")
        dm = bench_decode_multi(dc)
        _log(f"[bench] decode_multi verify {dm['verify']['us_per_call']:.1f} us, "
             f"commit {dm['commit']['us_per_call']:.1f} us")
        result["decode_multi"] = dm

    if not args.no_varlen:
        vc = W.VARLEN_CONFIGS["varlen"]
        _log(f"[bench] varlen {vc.describe()}")
        vl = bench_varlen(vc)
        _log(f"[bench] varlen {vl['ckpt']['us_per_call']:.1f} us with checkpoints, "
             f"{vl['no_ckpt']['us_per_call']:.1f} us without")
        result["varlen"] = vl

    if not args.no_layer:
        _log("[bench] layer form (prologue + epilogue)")
        ly = bench_layer(W.PREFILL_CONFIGS["prefill"])
        _log("[bench] layer " + ", ".join(
            f"{n} {ly[n]['us_per_call']:.1f} us" for n in ("plain", "bounded_l2_normgate",
                                                          "scalar_gate_l2")) +
             f"; decode plain {ly['decode']['plain_us']:.1f} us, layer "
             f"{ly['decode']['bounded_l2_normgate_us']:.1f} us")
        result["layer"] = ly

    if not args.no_cpu:
        _log("[bench] cpu oracle baseline")
        # the CPU share this process may use (OMP_NUM_THREADS when set), which
        # can be smaller than the machine's core count
        cores = min(os.cpu_count() or 1, int(os.environ.get("OMP_NUM_THREADS", "0") or 0)
                    or (os.cpu_count() or 1))
        result["cpu_baseline"] = cpu_baseline_prefill(cfg, max_heads=cores)

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
