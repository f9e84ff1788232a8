"""Seeded sweep of prefill shapes through the C ABI against the fp64 oracle.

The case list is drawn once from a fixed seed, so every run checks the same
cases. It spans the kernel paths by sequence-head count (prep + state walk
with 16- and 32-column workgroups, the fused kernel with 64- and 128-column
workgroups), ragged and empty sequences, chunk sizes 16 to 64, both decay
distributions of the configurations, with and without an initial state, and
fp32 inputs with small head dimensions on the generic kernel. Packed calls
draw mixed lengths (empty and one-token sequences included) with and without
checkpoints, some of them with enough sequence-heads for the split schedule.
"""
import dataclasses
import random

import pytest
import torch

import gated_delta_rule_22_amd as kda
import oracle
import workloads as W
from gpu_helpers import TOL_BF16, TOL_F32, report, to_dev

pytestmark = pytest.mark.gpu


def _prefill_cases():
    rng = random.Random(20261202)
    cases = []
    # bf16, dk = dv = 128: B x H picks the path (split below 128 sequence-heads,
    # 32-column walk above 32 of them; fused from 128, 128-column from 256)
    # (T short: empty, one token or one partial chunk, on three of them)
    for B, H, short in [(1, 1, False), (2, 3, True), (1, 17, False), (1, 40, False),
                        (3, 20, True), (2, 64, False), (1, 129, False), (1, 200, True),
                        (2, 130, False), (1, 260, False)]:
        T = rng.choice([0, 1, rng.randint(2, 63)]) if short else rng.randint(65, 520)
        base = rng.choice(["prefill", "batched"])
        cases.append(("bf16", base, B, T, H, 128, 128, 64, rng.randint(0, 10_000)))
    # fp32 on the generic kernel: small and mixed head dimensions, chunk sizes
    for dk, dv, chunk in [(16, 16, 16), (32, 64, 32), (64, 32, 64), (128, 128, 32)]:
        B, H, T = rng.randint(1, 3), rng.randint(1, 5), rng.randint(0, 300)
        cases.append(("f32", "cpu", B, T, H, dk, dv, chunk, rng.randint(0, 10_000)))
    return cases


def _case_id(c):
    return f"{c[0]}-{c[1]}-B{c[2]}T{c[3]}H{c[4]}-d{c[5]}x{c[6]}-C{c[7]}"


@pytest.mark.parametrize("case", _prefill_cases(), ids=_case_id)
def test_prefill_random_shape(case):
    kind, base, B, T, H, dk, dv, chunk, seed = case
    cfg = dataclasses.replace(W.PREFILL_CONFIGS[base], dk=dk, dv=dv)
    x = W.prefill_inputs(cfg, B=B, T=T, H=H, seed=seed)
    xd = to_dev(x)
    o, S = kda.kda_prefill_fwd(xd["q"], xd["k"], xd["v"], xd["log_alpha"], xd["beta"], xd["S0"],
                               chunk=chunk)
    torch.cuda.synchronize()
    ro, rS = oracle.prefill_f64(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["S0"])
    report(f"random prefill {_case_id(case)}", [("o", o, ro), ("S", S, rS)],
           TOL_F32 if kind == "f32" else TOL_BF16)


def _varlen_cases():
    rng = random.Random(7_2026)
    cases = []
    # (sequences, heads, checkpoint interval); 16 x 16 and 12 x 24 sequence-heads
    # reach the split schedule (256 or more), the others the prep + walk or
    # the fused kernel on a table
    for N, H, ck in [(3, 2, 64), (7, 8, 0), (5, 30, 128), (16, 16, 256), (12, 24, 64)]:
        lengths = [rng.choice([0, 1, rng.randint(2, 200), rng.randint(200, 900)])
                   for _ in range(N)]
        if N * H >= 256:
            lengths[rng.randrange(N)] = rng.randint(1500, 2600)   # one long enough to split
        cases.append((N, H, ck, lengths, rng.randint(0, 10_000)))
    return cases


@pytest.mark.parametrize("case", _varlen_cases(), ids=lambda c: f"N{c[0]}H{c[1]}ck{c[2]}")
def test_varlen_random_lengths(case):
    N, H, ck, lengths, seed = case
    x = W.varlen_inputs(W.PREFILL_CONFIGS["batched"], lengths, H=H, seed=seed)
    xd = to_dev(x)
    o, S, Sc = kda.kda_prefill_varlen(xd["q"], xd["k"], xd["v"], xd["log_alpha"], xd["beta"],
                                      xd["cu_seqlens"], xd["S0"], ckpt_every=ck)
    torch.cuda.synchronize()
    ro, rS, rSc = oracle.prefill_varlen_f64(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"],
                                            x["cu_seqlens"], x["S0"], ckpt_every=ck)
    pairs = [("o", o, ro, (1,)), ("S_final", S, rS)]
    if rSc.shape[0]:
        pairs.append(("S_ckpt", Sc[:rSc.shape[0]], rSc))
    report(f"random varlen N{N} H{H} lengths {lengths} ckpt {ck}", pairs, TOL_BF16)
