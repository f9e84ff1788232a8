"""Calls captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

The allocation-free prefill exists for callers that cannot allocate, such as
code under graph capture; a decode step is the other call a serving loop
would capture. Neither issues a memset. Each graph is replayed several
times, with eager work (the outputs cleared, the state reset) and a
synchronisation between replays, and every replay must equal the eager call
bit for bit.
"""
import pytest
import torch

import gated_delta_rule_22_amd as kda
import workloads as W
from gpu_helpers import DEV

pytestmark = pytest.mark.gpu

REPLAYS = 4


def _capture(call):
    """Warm up on a side stream, then capture one call."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    return g


def test_noalloc_prefill_replays():
    c = W.PREFILL_CONFIGS["prefill"]              # 16 heads: prep + walk on the static scratch
    x = W.prefill_inputs(c, seed=91, device=DEV)
    o = torch.empty_like(x["v"])
    S = torch.empty((c.B, c.H, c.dk, c.dv), dtype=torch.float32, device=DEV)

    def call():
        kda.kda_prefill_fwd_noalloc(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["S0"],
                                    o, S)
    call()
    torch.cuda.synchronize()
    ro, rS = o.clone(), S.clone()
    g = _capture(call)
    for i in range(REPLAYS):
        o.zero_()
        S.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, ro), f"replay {i}: o differs from the eager call"
        assert torch.equal(S, rS), f"replay {i}: S_final differs from the eager call"


def test_decode_step_replays():
    dc = W.DECODE_CONFIGS["decode"]
    S0 = W.decode_state(dc, device=DEV)
    st = W.decode_step_inputs(dc, 3, device=DEV)
    S = S0.clone()
    o = torch.empty((dc.B, dc.H, dc.dv), dtype=dc.dtype, device=DEV)

    def call():
        kda.kda_decode_step(st["q"], st["k"], st["v"], st["log_alpha"], st["beta"], S, o=o)
    call()
    torch.cuda.synchronize()
    ro, rS = o.clone(), S.clone()
    S.copy_(S0)
    g = _capture(call)
    for i in range(REPLAYS):
        S.copy_(S0)                                   # each replay steps from S0
        o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, ro), f"replay {i}: o differs from the eager step"
        assert torch.equal(S, rS), f"replay {i}: S differs from the eager step"
