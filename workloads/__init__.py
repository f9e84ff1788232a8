"""Seeded synthetic inputs for the KDA prefill and decode workloads.

This module only draws random tensors; it holds none of the recurrence's
arithmetic, so the GPU path and the fp64 oracle can both consume its output
without sharing any computation.

Shapes and distributions follow the KDA layer described on the Kimi K3 pages:
per-head q, k in R^{d_k} and v in R^{d_v} ("Kimi K3" blog, section "Kimi Delta
Attention"); q and k are L2-normalised as the Kimi Linear layer does before the
recurrence ("Kimi K3: the manos...", section "Kimi Linear"); the per-channel
log-decay stays inside (-5, 0) ("LLM architecture at trillion scale", section 4,
the numerics note on the log-decay bound).

Layouts (row-major, contiguous):
    q, k       [B, T, H, d_k]   (bf16 or fp32)
    v          [B, T, H, d_v]   (bf16 or fp32)
    log_alpha  [B, T, H, d_k]   fp32, natural log of the per-channel decay
    beta       [B, T, H]        fp32
    S0         [B, H, d_k, d_v] fp32 or None (zeros)
Decode tensors drop the T axis.

Draw order for one generator seed: q, k, v, log_alpha, beta, S0.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch

__all__ = [
    "PrefillConfig", "DecodeConfig", "PREFILL_CONFIGS", "DECODE_CONFIGS",
    "prefill_inputs", "prefill_inputs_per_head", "prefill_inputs_by_head", "decode_state",
    "decode_step_inputs",
    "VarlenConfig", "VARLEN_CONFIGS", "varlen_lengths", "varlen_inputs", "layer_inputs",
]


@dataclasses.dataclass(frozen=True)
class PrefillConfig:
    name: str
    B: int
    T: int
    H: int
    dk: int
    dv: int
    dtype: torch.dtype
    la_kind: str          # "uniform": -U(lo, hi); "softplus": -softplus(N(lo, hi))
    la_lo: float
    la_hi: float
    beta_kind: str        # "uniform": U(0,1); "sigmoid": sigmoid(N(0,1))
    s0_std: float         # 0 => S0 is None (zeros)
    chunk: int
    seed: int

    def describe(self) -> str:
        dt = "bf16" if self.dtype == torch.bfloat16 else "fp32"
        return (f"kda_prefill B{self.B} H{self.H} T{self.T} dk{self.dk} dv{self.dv} "
                f"C{self.chunk} {dt}")


@dataclasses.dataclass(frozen=True)
class DecodeConfig:
    name: str
    B: int
    H: int
    dk: int
    dv: int
    steps: int
    dtype: torch.dtype
    la_lo: float
    la_hi: float
    s_std: float
    seed: int

    def describe(self) -> str:
        dt = "bf16" if self.dtype == torch.bfloat16 else "fp32"
        return f"kda_decode B{self.B} H{self.H} dk{self.dk} dv{self.dv} {self.steps} steps {dt}"


PREFILL_CONFIGS = {
    # CPU-sized fp32 case.
    "cpu": PrefillConfig("cpu", 1, 64, 2, 16, 16, torch.float32,
                         "uniform", 0.001, 0.2, "uniform", 0.0, 16, 1),
    # Single-sequence prefill, 16 heads, 4K tokens.
    "prefill": PrefillConfig("prefill", 1, 4096, 16, 128, 128, torch.bfloat16,
                             "uniform", 0.001, 0.1, "sigmoid", 0.0, 64, 2),
    # Batched prefill with a carried initial state.
    "batched": PrefillConfig("batched", 8, 8192, 32, 128, 128, torch.bfloat16,
                             "softplus", -3.0, 1.0, "sigmoid", 0.02, 64, 3),
    # 1M-token context, 16384 chunks per head.
    "long": PrefillConfig("long", 1, 1 << 20, 32, 128, 128, torch.bfloat16,
                          "uniform", 0.0001, 0.05, "sigmoid", 0.0, 64, 4_000_000),
}

DECODE_CONFIGS = {
    "decode": DecodeConfig("decode", 256, 32, 128, 128, 1024, torch.bfloat16,
                           0.001, 0.1, 0.02, 5),
}


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _unit_rows(x: torch.Tensor) -> torch.Tensor:
    # L2-normalise over the last axis in fp32 (input recipe, not part of the op).
    return x / x.norm(dim=-1, keepdim=True).clamp_min(1e-12)


def _log_alpha(shape, kind, lo, hi, g, device):
    if kind == "uniform":
        u = torch.rand(shape, generator=g, device=device, dtype=torch.float32)
        return -(lo + (hi - lo) * u)
    if kind == "softplus":
        n = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        return -torch.nn.functional.softplus(lo + hi * n)
    raise ValueError(kind)


def _beta(shape, kind, g, device):
    if kind == "uniform":
        return torch.rand(shape, generator=g, device=device, dtype=torch.float32)
    if kind == "sigmoid":
        return torch.sigmoid(torch.randn(shape, generator=g, device=device,
                                         dtype=torch.float32))
    raise ValueError(kind)


def prefill_inputs(cfg: PrefillConfig, *, B: Optional[int] = None, T: Optional[int] = None,
                   H: Optional[int] = None, seed: Optional[int] = None,
                   device="cpu", dtype: Optional[torch.dtype] = None) -> dict:
    """Draw one prefill batch. Overrides let tests reuse a config's
    distributions at other sizes (ragged T, fewer heads)."""
    B = cfg.B if B is None else B
    T = cfg.T if T is None else T
    H = cfg.H if H is None else H
    dtype = cfg.dtype if dtype is None else dtype
    seed = cfg.seed if seed is None else seed
    g = _gen(seed, device)
    dk, dv = cfg.dk, cfg.dv
    q = _unit_rows(torch.randn((B, T, H, dk), generator=g, device=device)).to(dtype)
    k = _unit_rows(torch.randn((B, T, H, dk), generator=g, device=device)).to(dtype)
    v = torch.randn((B, T, H, dv), generator=g, device=device).to(dtype)
    la = _log_alpha((B, T, H, dk), cfg.la_kind, cfg.la_lo, cfg.la_hi, g, device)
    beta = _beta((B, T, H), cfg.beta_kind, g, device)
    S0 = None
    if cfg.s0_std > 0:
        S0 = cfg.s0_std * torch.randn((B, H, dk, dv), generator=g, device=device)
    return dict(q=q, k=k, v=v, log_alpha=la, beta=beta, S0=S0)


def prefill_inputs_per_head(cfg: PrefillConfig, h: int, *, T: Optional[int] = None,
                            device="cpu", dtype: Optional[torch.dtype] = None) -> dict:
    """One head's slice (B=1) drawn from its own seed cfg.seed + h, so a long
    context can be built head by head and any head regenerated alone.
    Shapes are [1, T, 1, d] / [1, T, 1] / [1, 1, dk, dv]."""
    return prefill_inputs(cfg, B=1, T=T, H=1, seed=cfg.seed + h, device=device, dtype=dtype)


def prefill_inputs_by_head(cfg: PrefillConfig, *, T: Optional[int] = None, device="cpu") -> dict:
    """A single-sequence batch (B = 1) assembled from per-head draws
    (prefill_inputs_per_head for h = 0..H-1), so that any head of a long
    context can later be regenerated alone. Shapes as prefill_inputs."""
    assert cfg.B == 1 and cfg.s0_std == 0, "per-head draws are defined for B = 1, S0 = 0"
    T = cfg.T if T is None else T
    H, dk, dv = cfg.H, cfg.dk, cfg.dv
    out = dict(q=torch.empty((1, T, H, dk), dtype=cfg.dtype, device=device),
               k=torch.empty((1, T, H, dk), dtype=cfg.dtype, device=device),
               v=torch.empty((1, T, H, dv), dtype=cfg.dtype, device=device),
               log_alpha=torch.empty((1, T, H, dk), dtype=torch.float32, device=device),
               beta=torch.empty((1, T, H), dtype=torch.float32, device=device), S0=None)
    for h in range(H):
        xh = prefill_inputs_per_head(cfg, h, T=T, device=device)
        for n in ("q", "k", "v", "log_alpha", "beta"):
            out[n][:, :, h] = xh[n][:, :, 0]
        del xh
    return out


def decode_state(cfg: DecodeConfig, device="cpu") -> torch.Tensor:
    g = _gen(cfg.seed, device)
    return cfg.s_std * torch.randn((cfg.B, cfg.H, cfg.dk, cfg.dv), generator=g, device=device)


def decode_step_inputs(cfg: DecodeConfig, step: int, *, B: Optional[int] = None,
                       device="cpu") -> dict:
    """Inputs of one decode step, drawn from seed 5_000_000 + step."""
    B = cfg.B if B is None else B
    g = _gen(5_000_000 + step, device)
    H, dk, dv = cfg.H, cfg.dk, cfg.dv
    q = _unit_rows(torch.randn((B, H, dk), generator=g, device=device)).to(cfg.dtype)
    k = _unit_rows(torch.randn((B, H, dk), generator=g, device=device)).to(cfg.dtype)
    v = torch.randn((B, H, dv), generator=g, device=device).to(cfg.dtype)
    la = _log_alpha((B, H, dk), "uniform", cfg.la_lo, cfg.la_hi, g, device)
    beta = _beta((B, H), "sigmoid", g, device)
    return dict(q=q, k=k, v=v, log_alpha=la, beta=beta)


@dataclasses.dataclass(frozen=True)
class VarlenConfig:
    """A packed batch of prompts of mixed lengths (serving prefill): lengths
    log-uniform in [len_lo, len_hi] until `total` tokens, state checkpoints
    every `ckpt_every` tokens of each prompt (the 512-token prefix-cache grid
    on the trillion-scale architecture page, section 6). Per-token
    distributions come from the prefill config `base`."""
    name: str
    total: int
    H: int
    len_lo: int
    len_hi: int
    ckpt_every: int
    base: str
    seed: int

    def describe(self) -> str:
        return (f"kda_prefill_varlen T{self.total} H{self.H} lengths {self.len_lo}.."
                f"{self.len_hi} ckpt {self.ckpt_every} bf16")


VARLEN_CONFIGS = {
    # The batched configuration's 65,536 tokens per 32 heads, as a mix of
    # prompt lengths instead of eight equal sequences.
    "varlen": VarlenConfig("varlen", 65536, 32, 256, 16384, 512, "batched", 11),
}


def varlen_lengths(total: int, lo: int, hi: int, seed: int) -> list:
    """Sequence lengths, log-uniform in [lo, hi], summing to exactly `total`
    (the last one is cut to fit)."""
    g = _gen(seed, "cpu")
    out, acc = [], 0
    while acc < total:
        u = float(torch.rand((), generator=g))
        n = int(round(lo * (hi / lo) ** u))
        n = min(max(n, 1), total - acc)
        out.append(n)
        acc += n
    return out


def varlen_inputs(base: PrefillConfig, lengths, *, H: Optional[int] = None,
                  seed: Optional[int] = None, device="cpu",
                  dtype: Optional[torch.dtype] = None) -> dict:
    """Packed inputs for sequences of the given lengths: q, k, log_alpha
    [T, H, dk], v [T, H, dv], beta [T, H], S0 [N, H, dk, dv] (or None), and
    cu_seqlens int32 [N + 1] on the CPU."""
    T = int(sum(lengths))
    N = len(lengths)
    x = prefill_inputs(base, B=1, T=T, H=H, seed=seed, device=device, dtype=dtype)
    out = {n: x[n][0] for n in ("q", "k", "v", "log_alpha", "beta")}
    H_ = out["q"].shape[1]
    S0 = None
    if base.s0_std > 0:
        g = _gen((base.seed if seed is None else seed) + 7_000_000, device)
        S0 = base.s0_std * torch.randn((N, H_, base.dk, base.dv), generator=g, device=device)
    out["S0"] = S0
    cu = [0]
    for n in lengths:
        cu.append(cu[-1] + int(n))
    out["cu_seqlens"] = torch.tensor(cu, dtype=torch.int32)
    return out


def layer_inputs(cfg: PrefillConfig, *, B: Optional[int] = None, T: Optional[int] = None,
                 H: Optional[int] = None, seed: Optional[int] = None, device="cpu",
                 dtype: Optional[torch.dtype] = None, decode: bool = False) -> dict:
    """Inputs of the layer form (weight-free prologue and epilogue around the
    op), as the projections would hand them over: raw q, k ~ N(0, 1) (not
    normalised), the decay gate pre-activation g ~ N(-5, 1.5) per key channel
    (so -5 sigmoid(g) is mostly a mild decay, with a tail of strong ones), a
    scalar per-head log-decay a = -U(lo, hi) of the config for the Gated
    DeltaNet form, beta as the config draws it, the output gate
    pre-activation z ~ N(0, 1) and an RMS-norm weight w = 1 + 0.1 N(0, 1)
    (fp32, [dv]). q, k, v, g, z in `dtype`; a, beta, w fp32. decode=True drops
    the T axis (T = 1)."""
    B = cfg.B if B is None else B
    T = 1 if decode else (cfg.T if T is None else T)
    H = cfg.H if H is None else H
    dtype = cfg.dtype if dtype is None else dtype
    seed = (cfg.seed if seed is None else seed) + 9_000_000
    g = _gen(seed, device)
    dk, dv = cfg.dk, cfg.dv
    shp = (B, T, H)
    out = dict(
        q=torch.randn(shp + (dk,), generator=g, device=device).to(dtype),
        k=torch.randn(shp + (dk,), generator=g, device=device).to(dtype),
        v=torch.randn(shp + (dv,), generator=g, device=device).to(dtype),
        g=(torch.randn(shp + (dk,), generator=g, device=device) * 1.5 - 5.0).to(dtype),
        a=-(0.001 + 0.099 * torch.rand(shp, generator=g, device=device)),
        beta=torch.sigmoid(torch.randn(shp, generator=g, device=device)),
        z=torch.randn(shp + (dv,), generator=g, device=device).to(dtype),
        w=1.0 + 0.1 * torch.randn((dv,), generator=g, device=device),
    )
    out["S0"] = None
    if cfg.s0_std > 0:
        out["S0"] = cfg.s0_std * torch.randn((B, H, dk, dv), generator=g, device=device)
    if decode:
        for n in ("q", "k", "v", "g", "a", "beta", "z"):
            out[n] = out[n][:, 0]
    return out
