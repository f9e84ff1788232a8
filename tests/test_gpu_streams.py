"""Calls on a stream other than the current one, through the C ABI.

The binding allocates what the caller leaves out (outputs, the workspace) with
torch, whose caching allocator ties memory to the current stream. A call on
another stream must keep that memory from being handed out again while its
kernels still run there. Each case launches on a side stream, at once
allocates and fills a buffer of the workspace's size on the current stream
(the block a premature release would give back), and then checks the results
against the fp64 oracle.
"""
import dataclasses

import pytest
import torch

import gated_delta_rule_22_amd as kda
import oracle
import workloads as W
from gpu_helpers import DEV, TOL_BF16, report, to_dev

pytestmark = pytest.mark.gpu


def _on_side_stream(call, junk_bytes):
    cur = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side.wait_stream(cur)                          # the inputs are ready
    out = call(side)
    junk = torch.empty(max(junk_bytes, 1), dtype=torch.uint8, device=DEV)
    junk.fill_(0xFF)                               # NaN bit patterns in bf16 and fp32
    cur.wait_stream(side)
    torch.cuda.synchronize()
    del junk
    return out


def test_prefill_split_path_on_side_stream():
    c = W.PREFILL_CONFIGS["prefill"]              # 16 heads: prep + state walk, 74 MB workspace
    x = W.prefill_inputs(c, seed=77)
    xd = to_dev(x)
    wsb = kda.kda_prefill_workspace_size(c.B, c.T, c.H, c.dk, c.dv, c.dtype)
    assert wsb > 0
    o, S = _on_side_stream(lambda s: kda.kda_prefill_fwd(
        xd["q"], xd["k"], xd["v"], xd["log_alpha"], xd["beta"], xd["S0"], stream=s), wsb)
    ro, rS = oracle.prefill_f64(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["S0"])
    report("prefill B1 H16 T4096 on a side stream", [("o", o, ro), ("S", S, rS)], TOL_BF16)


def test_varlen_on_side_stream():
    lengths = [700, 0, 1, 1500, 64, 300]
    x = W.varlen_inputs(W.PREFILL_CONFIGS["batched"], lengths, H=8, seed=78)
    xd = to_dev(x)
    N, T = len(lengths), sum(lengths)
    wsb = kda.kda_prefill_varlen_workspace_size(N, T, 8, 128, 128, torch.bfloat16)
    o, S, Sc = _on_side_stream(lambda s: kda.kda_prefill_varlen(
        xd["q"], xd["k"], xd["v"], xd["log_alpha"], xd["beta"], xd["cu_seqlens"], xd["S0"],
        ckpt_every=128, stream=s), wsb)
    ro, rS, rSc = oracle.prefill_varlen_f64(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"],
                                            x["cu_seqlens"], x["S0"], ckpt_every=128)
    report("packed prefill on a side stream",
           [("o", o, ro, (1,)), ("S_final", S, rS), ("S_ckpt", Sc[:rSc.shape[0]], rSc)], TOL_BF16)


def test_decode_on_side_stream():
    dc = dataclasses.replace(W.DECODE_CONFIGS["decode"], B=8)
    S0 = W.decode_state(dc)
    st = W.decode_step_inputs(dc, 0)
    S = S0.to(DEV)
    sd = to_dev(st)
    o = _on_side_stream(lambda s: kda.kda_decode_step(
        sd["q"], sd["k"], sd["v"], sd["log_alpha"], sd["beta"], S, stream=s), 1 << 20)
    ro, rS = oracle.decode_f64(st["q"], st["k"], st["v"], st["log_alpha"], st["beta"], S0)
    report("decode step B8 H32 on a side stream", [("o", o, ro, (0, 1)), ("S", S, rS)], TOL_BF16)
