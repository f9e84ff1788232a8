"""GPU parity of the layer form (kda_prefill_layer, kda_decode_layer) through
the C ABI against the fp64 oracle's layer functions.

Every gate mode (given log-decay, bounded pre-activation, per-head scalar)
runs with and without in-kernel L2 normalisation and with and without the
output norm-gate epilogue, on each prefill path (prep + state walk, fused
with 64- and 128-column workgroups, fp32 generic) and on decode. With default
options both calls must be bit-identical to the plain entry points.
"""
import dataclasses
import itertools

import pytest
import torch

import gated_delta_rule_22_amd as kda
import oracle
from oracle import layer as OL
import workloads as W
from gpu_helpers import DEV, TOL_BF16, TOL_F32, report, to_dev

pytestmark = pytest.mark.gpu

BASE = W.PREFILL_CONFIGS["batched"]
MODES = {"log": kda.KDA_GATE_LOG, "bounded": kda.KDA_GATE_BOUNDED,
         "scalar": kda.KDA_GATE_SCALAR}


def gate_input(x, mode):
    """The gate tensor of a mode from one layer-input draw (the given
    log-decay of the log mode is -5 sigmoid(g) in fp32)."""
    if mode == "bounded":
        return x["g"]
    if mode == "scalar":
        return x["a"]
    return (-5.0 * torch.sigmoid(x["g"].float())).contiguous()


def unit_qk(x):
    """Without in-kernel normalisation the op needs unit-norm keys (raw keys
    of norm ~sqrt(dk) make I - beta k k^T expand and the state diverge)."""
    for n in ("q", "k"):
        t = x[n]
        x[n] = torch.nn.functional.normalize(t.float(), dim=-1).to(t.dtype)
    return x


def run_prefill(x, mode, l2, epi, chunk=64):
    if not l2:
        x = unit_qk(dict(x))
    xd = to_dev(x)
    o, S = kda.kda_prefill_layer(xd["q"], xd["k"], xd["v"], to_dev({"g": gate_input(x, mode)})["g"],
                                 xd["beta"], xd["S0"], gate_mode=MODES[mode], l2norm=l2,
                                 z=xd["z"] if epi else None, w=xd["w"] if epi else None,
                                 chunk=chunk)
    torch.cuda.synchronize()
    ro, rS = OL.layer_prefill_f64(x["q"], x["k"], x["v"], gate_input(x, mode), x["beta"],
                                  x["S0"], l2norm=l2, gate=MODES[mode],
                                  z=x["z"] if epi else None, w=x["w"] if epi else None)
    return (o, S), (ro, rS)


COMBOS = list(itertools.product(["log", "bounded", "scalar"], [False, True], [False, True]))


@pytest.mark.parametrize("mode,l2,epi", COMBOS)
def test_prefill_split_path_all_combos(mode, l2, epi):
    x = W.layer_inputs(BASE, B=1, T=200, H=4)
    (o, S), (ro, rS) = run_prefill(x, mode, l2, epi)
    report(f"layer prefill split {mode} l2={l2} epi={epi}", [("o", o, ro), ("S", S, rS)],
           TOL_BF16)


@pytest.mark.parametrize("B,H", [(2, 64), (4, 64)])   # fused, 64- and 128-column workgroups
@pytest.mark.parametrize("mode,l2,epi", [("bounded", True, True), ("scalar", True, False),
                                         ("log", False, True)])
def test_prefill_fused_paths(B, H, mode, l2, epi):
    x = W.layer_inputs(BASE, B=B, T=130, H=H)
    (o, S), (ro, rS) = run_prefill(x, mode, l2, epi)
    report(f"layer prefill fused B{B} H{H} {mode} l2={l2} epi={epi}",
           [("o", o, ro), ("S", S, rS)], TOL_BF16)


@pytest.mark.parametrize("mode,l2,epi", COMBOS)
def test_prefill_fp32_generic(mode, l2, epi):
    c = dataclasses.replace(BASE, dk=32, dv=64)
    x = W.layer_inputs(c, B=2, T=77, H=3, dtype=torch.float32)
    (o, S), (ro, rS) = run_prefill(x, mode, l2, epi, chunk=32)
    report(f"layer prefill fp32 {mode} l2={l2} epi={epi}", [("o", o, ro), ("S", S, rS)],
           TOL_F32)


def test_prefill_default_options_equal_plain_op():
    x = to_dev(W.prefill_inputs(BASE, B=1, T=300, H=4))
    o1, S1 = kda.kda_prefill_fwd(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["S0"])
    o2, S2 = kda.kda_prefill_layer(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["S0"])
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_prefill_layer_prefill_config_full():
    # the 4K-token, 16-head shape with the whole prologue and epilogue
    c = W.PREFILL_CONFIGS["prefill"]
    x = W.layer_inputs(c)
    (o, S), (ro, rS) = run_prefill(x, "bounded", True, True)
    report("layer prefill B1 H16 T4096 bounded+l2+epilogue", [("o", o, ro), ("S", S, rS)],
           TOL_BF16)


def run_decode(x, S0, mode, l2, epi):
    if not l2:
        x = unit_qk(dict(x))
    xd = to_dev(x)
    S = S0.to(DEV).clone()
    g = to_dev({"g": gate_input(x, mode)})["g"]
    o = kda.kda_decode_layer(xd["q"], xd["k"], xd["v"], g, xd["beta"], S, gate_mode=MODES[mode],
                             l2norm=l2, z=xd["z"] if epi else None, w=xd["w"] if epi else None)
    torch.cuda.synchronize()
    ro, rS = OL.layer_decode_f64(x["q"], x["k"], x["v"], gate_input(x, mode), x["beta"], S0,
                                 l2norm=l2, gate=MODES[mode], z=x["z"] if epi else None,
                                 w=x["w"] if epi else None)
    return (o, S), (ro, rS)


@pytest.mark.parametrize("mode,l2,epi", COMBOS)
def test_decode_fp32_all_combos(mode, l2, epi):
    c = dataclasses.replace(BASE, dk=64, dv=128)
    x = W.layer_inputs(c, B=3, H=5, dtype=torch.float32, decode=True)
    S0 = 0.1 * torch.randn((3, 5, 64, 128), generator=torch.Generator().manual_seed(5))
    (o, S), (ro, rS) = run_decode(x, S0, mode, l2, epi)
    report(f"layer decode fp32 {mode} l2={l2} epi={epi}", [("o", o, ro), ("S", S, rS)], TOL_F32)


@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 64), (128, 32), (16, 128)])
def test_decode_shapes(dk, dv):
    c = dataclasses.replace(BASE, dk=dk, dv=dv)
    x = W.layer_inputs(c, B=2, H=7, dtype=torch.float32, decode=True)
    S0 = 0.1 * torch.randn((2, 7, dk, dv), generator=torch.Generator().manual_seed(6))
    (o, S), (ro, rS) = run_decode(x, S0, "bounded", True, True)
    report(f"layer decode fp32 dk{dk} dv{dv}", [("o", o, ro), ("S", S, rS)], TOL_F32)


def test_decode_bf16_decode_config():
    dc = W.DECODE_CONFIGS["decode"]
    c = dataclasses.replace(BASE, dk=dc.dk, dv=dc.dv)
    x = W.layer_inputs(c, B=dc.B, H=dc.H, decode=True)
    S0 = W.decode_state(dc)
    (o, S), (ro, rS) = run_decode(x, S0, "bounded", True, True)
    report("layer decode bf16 B256 H32 bounded+l2+epilogue", [("o", o, ro), ("S", S, rS)],
           TOL_BF16)


def test_decode_default_options_equal_plain_step():
    dc = W.DECODE_CONFIGS["decode"]
    s = to_dev(W.decode_step_inputs(dc, 0, B=8))
    S0 = W.decode_state(dc)[:8].to(DEV)
    S1, S2 = S0.clone(), S0.clone()
    o1 = kda.kda_decode_step(s["q"], s["k"], s["v"], s["log_alpha"], s["beta"], S1)
    o2 = kda.kda_decode_layer(s["q"], s["k"], s["v"], s["log_alpha"], s["beta"], S2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
