"""Host-side checks of the seeded input generators and the flop/byte accounting."""
import torch

import workloads as W
from workloads import accounting as A


def test_accounting_matches_complexity_section():
    # "Kimi K3: the manos..." section "Complexity Analysis": per chunk-head
    # 12C^3 + 8C^2 D + 6C D^2 flops and 8C^2 + 22CD bytes.
    assert A.chunk_head_flops(64, 128) == 13_631_488
    assert A.two_kernel_chunk_bytes(64, 128) == 212_992
    # 7 D^2 flops and 8 D^2 state bytes per head per decode step
    assert A.decode_step_flops(1, 1, 128, 128) == 7 * 128 * 128
    assert A.decode_step_bytes(1, 1, 128, 128) - 8 * 128 * 128 == 2 * 3 * 128 + 4 * 128 + 4 + 2 * 128


def test_prefill_bytes_per_token_head():
    # q,k,v,o bf16 + log-decay fp32 + beta fp32 = 1540 B per token-head at D=128
    assert A.prefill_bytes(1, 1, 1, 128, 128, has_s0=False, writes_state=False) == 1540
    c = W.PREFILL_CONFIGS["prefill"]
    assert A.prefill_bytes(c.B, c.T, c.H, c.dk, c.dv, has_s0=False) == \
        1540 * 4096 * 16 + 16 * 4 * 128 * 128


def test_generators_are_seeded_and_shaped():
    c = W.PREFILL_CONFIGS["cpu"]
    a = W.prefill_inputs(c)
    b = W.prefill_inputs(c)
    for key in ("q", "k", "v", "log_alpha", "beta"):
        assert torch.equal(a[key], b[key]), key
    assert a["q"].shape == (1, 64, 2, 16) and a["q"].dtype == torch.float32
    assert a["beta"].shape == (1, 64, 2)
    assert a["S0"] is None
    n = a["q"].double().norm(dim=-1)
    assert torch.allclose(n, torch.ones_like(n), atol=1e-6)
    assert float(a["log_alpha"].max()) <= -0.001 and float(a["log_alpha"].min()) >= -0.2
    assert 0.0 <= float(a["beta"].min()) and float(a["beta"].max()) <= 1.0


def test_generator_overrides_and_bf16():
    c = W.PREFILL_CONFIGS["batched"]
    x = W.prefill_inputs(c, B=1, T=100, H=2)
    assert x["q"].dtype == torch.bfloat16 and x["q"].shape == (1, 100, 2, 128)
    assert x["S0"].shape == (1, 2, 128, 128)
    assert float(x["log_alpha"].max()) < 0.0
    h3 = W.prefill_inputs_per_head(W.PREFILL_CONFIGS["long"], 3, T=128)
    h3b = W.prefill_inputs_per_head(W.PREFILL_CONFIGS["long"], 3, T=128)
    assert torch.equal(h3["k"], h3b["k"]) and h3["k"].shape == (1, 128, 1, 128)


def test_decode_inputs():
    c = W.DECODE_CONFIGS["decode"]
    s = W.decode_step_inputs(c, 7, B=2)
    assert s["q"].shape == (2, 32, 128) and s["beta"].shape == (2, 32)
    assert torch.equal(s["v"], W.decode_step_inputs(c, 7, B=2)["v"])
