"""Identical calls return bit-identical results, for every entry point.

No kernel here uses atomics or reductions whose order depends on timing, so
any difference between two identical calls is a defect (a race, or a
hardware hazard the code does not respect). Each case runs three calls on
the same inputs and compares every output element by element; a packed
call's checkpoint buffer is compared over the slots it writes.
"""
import dataclasses

import pytest
import torch

import gated_delta_rule_22_amd as kda
import workloads as W
from gpu_helpers import DEV

pytestmark = pytest.mark.gpu

CALLS = 3


def _same(label, fn):
    first = None
    for i in range(CALLS):
        outs = [t.detach().clone() for t in fn() if t is not None]
        torch.cuda.synchronize()
        if first is None:
            first = outs
            continue
        for j, (a, b) in enumerate(zip(first, outs)):
            assert torch.equal(a, b), (f"{label}: output {j} of call {i} differs from call 0 in "
                                       f"{int((a != b).sum())} elements")


@pytest.mark.parametrize("B,T,H", [(1, 4096, 16), (1, 3000, 48), (2, 700, 64), (2, 1000, 256)])
def test_prefill_repeatable(B, T, H):
    # split path with 16- and 32-column walks, fused with 64 and 128 columns
    x = W.prefill_inputs(W.PREFILL_CONFIGS["batched"], B=B, T=T, H=H, device=DEV)
    _same(f"prefill B{B} T{T} H{H}",
          lambda: kda.kda_prefill_fwd(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["S0"]))


def test_batched_config_repeatable():
    # B8 H32 T8192 with carried state: the fused kernel at full size
    c = W.PREFILL_CONFIGS["batched"]
    x = W.prefill_inputs(c, device=DEV)
    _same("batched configuration B8 H32 T8192",
          lambda: kda.kda_prefill_fwd(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["S0"]))


def test_long_config_repeatable():
    # B1 H32 T1048576: 171 pieces of prep and state walk, every output element
    c = W.PREFILL_CONFIGS["long"]
    x = W.prefill_inputs_by_head(c, device=DEV)
    _same("1M-token configuration B1 H32",
          lambda: kda.kda_prefill_fwd(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], None))
    del x
    torch.cuda.empty_cache()


def test_piecewise_prefill_repeatable():
    c = W.PREFILL_CONFIGS["long"]
    x = W.prefill_inputs_by_head(c, T=1 << 17, device=DEV)
    _same("piecewise prefill B1 H32 T131072",
          lambda: kda.kda_prefill_fwd(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], None))


def test_varlen_repeatable():
    vc = W.VARLEN_CONFIGS["varlen"]
    lengths = W.varlen_lengths(vc.total, vc.len_lo, vc.len_hi, vc.seed)
    x = W.varlen_inputs(W.PREFILL_CONFIGS[vc.base], lengths, H=vc.H, seed=vc.seed, device=DEV)
    cu = x["cu_seqlens"].to(DEV)
    n_ck = sum(n // vc.ckpt_every for n in lengths)

    def call():
        o, S, Sc = kda.kda_prefill_varlen(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], cu,
                                          x["S0"], ckpt_every=vc.ckpt_every)
        return o, S, Sc[:n_ck]
    _same("packed 65,536-token mix, checkpoints every 512 tokens", call)


def test_decode_repeatable():
    dc = W.DECODE_CONFIGS["decode"]
    S0 = W.decode_state(dc, device=DEV)
    s = W.decode_step_inputs(dc, 0, device=DEV)

    def call():
        S = S0.clone()
        return kda.kda_decode_step(s["q"], s["k"], s["v"], s["log_alpha"], s["beta"], S), S
    _same("decode step B256 H32", call)


def test_decode_multi_repeatable():
    dc = W.DECODE_CONFIGS["decode"]
    S0 = W.decode_state(dc, device=DEV)
    x = W.prefill_inputs(dataclasses.replace(W.PREFILL_CONFIGS["prefill"]), B=dc.B, T=8, H=dc.H,
                         seed=dc.seed + 5, device=DEV)
    n = torch.randint(0, 9, (dc.B,), generator=torch.Generator().manual_seed(6))
    n = n.to(torch.int32).to(DEV)

    def call():
        S = S0.clone()
        return kda.kda_decode_multi(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], S,
                                    n_commit=n), S
    _same("8-token draft B256 H32, random accepted prefixes", call)


def test_layer_forms_repeatable():
    lx = W.layer_inputs(W.PREFILL_CONFIGS["prefill"], device=DEV)
    _same("layer prefill 4K, bounded gate + L2 + norm-gate", lambda: kda.kda_prefill_layer(
        lx["q"], lx["k"], lx["v"], lx["g"], lx["beta"], None, gate_mode=kda.KDA_GATE_BOUNDED,
        l2norm=True, z=lx["z"], w=lx["w"]))
    # 64 sequence-heads: split path and the separate epilogue kernel;
    # 256: the 128-column fused kernel with the epilogue in registers
    for B in (2, 8):
        lb = W.layer_inputs(W.PREFILL_CONFIGS["batched"], B=B, T=300, device=DEV)
        _same(f"layer prefill B{B} H32 T300", lambda: kda.kda_prefill_layer(
            lb["q"], lb["k"], lb["v"], lb["g"], lb["beta"], None, gate_mode=kda.KDA_GATE_BOUNDED,
            l2norm=True, z=lb["z"], w=lb["w"]))
    dc = W.DECODE_CONFIGS["decode"]
    S0 = W.decode_state(dc, device=DEV)
    ld = W.layer_inputs(dataclasses.replace(W.PREFILL_CONFIGS["prefill"]), B=dc.B, H=dc.H,
                        decode=True, device=DEV)

    def dec():
        S = S0.clone()
        return kda.kda_decode_layer(ld["q"], ld["k"], ld["v"], ld["g"], ld["beta"], S,
                                    gate_mode=kda.KDA_GATE_BOUNDED, l2norm=True, z=ld["z"],
                                    w=ld["w"]), S
    _same("layer decode B256 H32", dec)
