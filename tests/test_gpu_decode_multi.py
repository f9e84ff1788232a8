"""GPU parity of kda_decode_multi (through the C ABI) against the fp64 oracle.

The multi-token step runs T tokens from a live state, returns o for every
token and leaves S[b] at the state after the accepted prefix n_commit[b]. Its
plain definition is the token recurrence itself, so the reference is the
oracle's token loop: o over all T tokens from S0, and the state after the
first n_commit[b] tokens of sequence b.
"""
import dataclasses

import numpy as np
import pytest
import torch

import gated_delta_rule_22_amd as kda
import oracle
import workloads as W
from gpu_helpers import DEV, TOL_BF16, TOL_F32, report, to_dev

pytestmark = pytest.mark.gpu


def inputs(B, T, H, dk=128, dv=128, dtype=torch.bfloat16, seed=11):
    cfg = dataclasses.replace(W.PREFILL_CONFIGS["prefill"], dk=dk, dv=dv)
    x = W.prefill_inputs(cfg, B=B, T=T, H=H, seed=seed, dtype=dtype)
    g = torch.Generator().manual_seed(seed + 1)
    x["S0"] = 0.3 * torch.randn(B, H, dk, dv, generator=g)
    return x


def oracle_multi(x, n):
    """o over all T tokens; per sequence, the state after its first n[b] tokens."""
    ro, _ = oracle.prefill_f64(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["S0"])
    rS = np.zeros(tuple(x["S0"].shape), np.float64)
    for b, nb in enumerate(n):
        sl = {k: v[b:b + 1, :nb] for k, v in x.items() if k != "S0"}
        _, Sb = oracle.prefill_f64(sl["q"], sl["k"], sl["v"], sl["log_alpha"], sl["beta"],
                                   x["S0"][b:b + 1])
        rS[b] = Sb[0]
    return ro, rS


def gpu_multi(x, n=None):
    xd = to_dev({k: v for k, v in x.items() if k != "S0"})
    S = x["S0"].to(DEV).clone()
    nd = None if n is None else torch.tensor(n, dtype=torch.int32, device=DEV)
    o = kda.kda_decode_multi(xd["q"], xd["k"], xd["v"], xd["log_alpha"], xd["beta"], S,
                             n_commit=nd)
    torch.cuda.synchronize()
    return o, S


@pytest.mark.parametrize("dk,dv", [(16, 16), (16, 128), (128, 16), (64, 32), (128, 128)])
def test_multi_fp32_shapes(dk, dv):
    x = inputs(3, 5, 4, dk, dv, torch.float32, seed=dk + dv)
    n = [5, 0, 3]
    o, S = gpu_multi(x, n)
    ro, rS = oracle_multi(x, n)
    report(f"multi fp32 dk{dk} dv{dv} T5 n={n}", [("o", o, ro), ("S", S, rS)], TOL_F32)


@pytest.mark.parametrize("dtype,T", [(torch.bfloat16, 12), (torch.bfloat16, 33), (torch.float32, 20)])
def test_long_drafts_on_the_valu_kernel(dtype, T):
    # drafts past 8 tokens (and fp32 ones) take the VALU kernel
    B, H = 6, 8
    x = inputs(B, T, H, dtype=dtype, seed=40 + T)
    n = [int(v) for v in torch.randint(0, T + 1, (B,), generator=torch.Generator().manual_seed(T))]
    n[0], n[1] = 0, T
    o, S = gpu_multi(x, n)
    ro, rS = oracle_multi(x, n)
    report(f"multi {dtype} B{B} H{H} T{T} n={n}", [("o", o, ro), ("S", S, rS)],
           TOL_F32 if dtype == torch.float32 else TOL_BF16)


def test_multi_bf16_random_accept():
    B, T, H = 8, 8, 32
    x = inputs(B, T, H, seed=21)
    n = [int(v) for v in torch.randint(0, T + 1, (B,), generator=torch.Generator().manual_seed(3))]
    o, S = gpu_multi(x, n)
    ro, rS = oracle_multi(x, n)
    report(f"multi bf16 B{B} H{H} T{T} n={n}", [("o", o, ro), ("S", S, rS)], TOL_BF16)


def test_multi_bf16_decay_past_the_bound():
    # Log-decays of -8 to -20 per step on some channels and tokens, outside
    # the supported [-5, 0]: the matrix-core draft kernel clamps them to -10
    # (keeping exp(-10) of the old state), so it stays finite and within the
    # bf16 tolerance of the exact recurrence.
    B, T, H = 4, 8, 8
    x = inputs(B, T, H, seed=23)
    g = torch.Generator().manual_seed(24)
    x["log_alpha"][:, :, :, :16] = -8.0 - 12.0 * torch.rand(B, T, H, 16, generator=g)
    x["log_alpha"][:, 5] = -8.0 - 12.0 * torch.rand(B, H, 128, generator=g)
    n = [8, 3, 0, 6]
    o, S = gpu_multi(x, n)
    assert torch.isfinite(o.float()).all() and torch.isfinite(S).all()
    ro, rS = oracle_multi(x, n)
    report(f"multi bf16 log-decay -8..-20 B{B} H{H} T{T} n={n}", [("o", o, ro), ("S", S, rS)],
           TOL_BF16)


def test_verify_leaves_state_untouched():
    x = inputs(4, 6, 8, seed=31)
    o, S = gpu_multi(x, [0, 0, 0, 0])
    assert torch.equal(S.cpu(), x["S0"]), "a verify pass (n_commit = 0) must not write S"
    ro, _ = oracle_multi(x, [0, 0, 0, 0])
    report("verify only B4 H8 T6", [("o", o, ro)], TOL_BF16)


def test_out_of_range_counts_are_clamped():
    x = inputs(3, 4, 8, seed=41)
    o1, S1 = gpu_multi(x, [-3, 9, 2])
    o2, S2 = gpu_multi(x, [0, 4, 2])
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_null_commit_is_all_tokens():
    x = inputs(2, 5, 8, seed=51)
    o1, S1 = gpu_multi(x, None)
    o2, S2 = gpu_multi(x, [5, 5])
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_one_token_equals_decode_step():
    x = inputs(4, 1, 16, seed=61)
    o1, S1 = gpu_multi(x, None)
    xd = to_dev({k: v[:, 0] for k, v in x.items() if k != "S0"})
    S2 = x["S0"].to(DEV).clone()
    o2 = kda.kda_decode_step(xd["q"], xd["k"], xd["v"], xd["log_alpha"], xd["beta"], S2)
    torch.cuda.synchronize()
    assert torch.equal(o1[:, 0], o2) and torch.equal(S1, S2)


def test_verify_then_commit_equals_single_call():
    x = inputs(4, 7, 8, seed=71)
    n = [7, 2, 0, 5]
    o_verify, S_verify = gpu_multi(x, [0, 0, 0, 0])
    o_one, S_one = gpu_multi(x, n)
    assert torch.equal(o_verify, o_one), "o must not depend on the accepted count"
    assert torch.equal(S_verify.cpu(), x["S0"])
    # commit = the same call on the live state with the accepted counts
    ro, rS = oracle_multi(x, n)
    report(f"commit n={n}", [("o", o_one, ro), ("S", S_one, rS)], TOL_BF16)


def test_decode_config_size_draft():
    # the decode configuration (B256 H32 d128, fp32 state of 537 MB) with an
    # 8-token draft and random accepted prefixes; sampled sequences against
    # the oracle, and the first token of every head against one oracle step
    c = W.DECODE_CONFIGS["decode"]
    B, H, T = c.B, c.H, 8
    S0 = W.decode_state(c, device=DEV)
    cfg = dataclasses.replace(W.PREFILL_CONFIGS["prefill"])
    x = W.prefill_inputs(cfg, B=B, T=T, H=H, seed=81, device=DEV)
    n = torch.randint(0, T + 1, (B,), generator=torch.Generator().manual_seed(4))
    S = S0.clone()
    o = kda.kda_decode_multi(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], S,
                             n_commit=n.to(torch.int32).to(DEV))
    torch.cuda.synchronize()
    ro0, rS0 = oracle.decode_f64(x["q"][:, 0].cpu(), x["k"][:, 0].cpu(), x["v"][:, 0].cpu(),
                                 x["log_alpha"][:, 0].cpu(), x["beta"][:, 0].cpu(), S0.cpu())
    report("draft config, token 0, all 8192 heads", [("o", o[:, 0], ro0)], TOL_BF16)
    for b in (0, 97, 255):
        xb = {k: v[b:b + 1].cpu() for k, v in x.items() if v is not None}
        xb["S0"] = S0[b:b + 1].cpu()
        nb = int(n[b])
        ro, rS = oracle_multi(xb, [nb])
        report(f"draft config sequence {b} (n={nb})", [("o", o[b:b + 1], ro), ("S", S[b:b + 1], rS)],
               TOL_BF16)


@pytest.mark.parametrize("T", [2, 3])
def test_short_drafts_on_matrix_cores(T):
    # the bf16 d = 128 draft path for the shortest drafts, accepted counts
    # from 0 (verify only) to T
    B, H = 6, 16
    x = inputs(B, T, H, seed=90 + T)
    n = [0, 1, T, 1, T - 1, T]
    o, S = gpu_multi(x, n)
    ro, rS = oracle_multi(x, n)
    report(f"multi bf16 B{B} H{H} T{T} n={n}", [("o", o, ro), ("S", S, rS)], TOL_BF16)
    assert torch.equal(S[0].cpu(), x["S0"][0]), "n_commit = 0 must leave the state untouched"


def test_full_commit_every_head_repeated():
    # The decode configuration's state with an 8-token draft committed in
    # full, four times from the same state: every head against the oracle
    # each time, and the four results bit-identical (the kernel has no
    # atomics or reductions across workgroups, so any difference between
    # identical calls is a defect). A committing pass that turned its tiles
    # back into row pieces by lane permutes left stale values in a few heads
    # of most calls (rel-L2 up to about 0.1 against the 2.6e-3 of the rest);
    # the per-head bound here is 1e-2, four times the worst head measured
    # otherwise.
    c = W.DECODE_CONFIGS["decode"]
    B, H, T = c.B, c.H, 8
    S0 = W.decode_state(c, device=DEV)
    x = W.prefill_inputs(dataclasses.replace(W.PREFILL_CONFIGS["prefill"]), B=B, T=T, H=H,
                         seed=c.seed + 77, device=DEV)
    full = torch.full((B,), T, dtype=torch.int32, device=DEV)
    xc = {k: v.cpu() for k, v in x.items() if v is not None}
    ro, rS = oracle.prefill_f64(xc["q"], xc["k"], xc["v"], xc["log_alpha"], xc["beta"], S0.cpu())
    first = None
    for i in range(4):
        S = S0.clone()
        o = kda.kda_decode_multi(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], S,
                                 n_commit=full)
        torch.cuda.synchronize()
        report(f"full commit B{B} H{H} T{T}, call {i}", [("o", o, ro, (0, 2)), ("S", S, rS)], 1e-2)
        if first is None:
            first = (o.cpu(), S.cpu())
        else:
            assert torch.equal(o.cpu(), first[0]), f"call {i}: o differs from call 0"
            assert torch.equal(S.cpu(), first[1]), f"call {i}: S differs from call 0"
