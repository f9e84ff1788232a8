"""Algorithmic flop and byte counts for KDA prefill and decode.

These are the method's own work, not whatever a given kernel happens to do.

Prefill flops per chunk of C tokens and one head (d_k = d_v = D), as counted in
"Kimi K3: the manos..." section "Complexity Analysis": the chunk-prep part
(L, the Neumann-factorised inverse as six C x C x C products, M_qk) plus the
chunk-recurrent part (K_decay S, Q_decay S, M_qk U, INV B, K_restore^T U):
    12 C^3 + 8 C^2 D + 6 C D^2.
``prefill_flops_conservative`` drops the inverse (its cost depends on the method).

The same section counts ~7 D^2 flops and ~8 D^2 bytes (fp32 state read + write)
per head per decode step, and 8 C^2 + 22 C D bytes per chunk-head for a
two-kernel chunked prefill that stages its intermediates in HBM.

``prefill_bytes`` is the unavoidable HBM traffic of a single pass: q, k, v read
and o written in the activation dtype, the fp32 log-decay and beta read, and the
fp32 state read once (S0) and written once (S_final).
"""
from __future__ import annotations

import math


def chunk_head_flops(C: int, D: int) -> int:
    return 12 * C**3 + 8 * C**2 * D + 6 * C * D**2


def chunk_head_flops_conservative(C: int, D: int) -> int:
    return 8 * C**2 * D + 6 * C * D**2


def two_kernel_chunk_bytes(C: int, D: int) -> int:
    """Bytes per chunk-head of the two-kernel staged scheme (2-byte elements)."""
    return 8 * C**2 + 22 * C * D


def prefill_flops(B: int, T: int, H: int, D: int, C: int) -> int:
    return B * H * math.ceil(T / C) * chunk_head_flops(C, D)


def prefill_flops_conservative(B: int, T: int, H: int, D: int, C: int) -> int:
    return B * H * math.ceil(T / C) * chunk_head_flops_conservative(C, D)


def prefill_bytes(B: int, T: int, H: int, dk: int, dv: int, elt: int = 2,
                  has_s0: bool = True, writes_state: bool = True) -> int:
    per_token_head = elt * (2 * dk + dv) + 4 * dk + 4 + elt * dv
    state = 4 * dk * dv * (int(has_s0) + int(writes_state))
    return B * T * H * per_token_head + B * H * state


def decode_step_bytes(B: int, H: int, dk: int, dv: int, elt: int = 2) -> int:
    return B * H * (8 * dk * dv + elt * (2 * dk + dv) + 4 * dk + 4 + elt * dv)


def decode_multi_bytes(B: int, H: int, T: int, dk: int, dv: int, commit: bool,
                       elt: int = 2) -> int:
    """Multi-token decode: the fp32 state read once (and written once when a
    prefix is committed) plus T tokens of q, k, v, o, log-decay and beta."""
    state = 4 * dk * dv * (2 if commit else 1)
    per_token = elt * (2 * dk + dv) + 4 * dk + 4 + elt * dv
    return B * H * (state + T * per_token)


def decode_step_flops(B: int, H: int, dk: int, dv: int) -> int:
    return 7 * dk * dv * B * H


def oracle_flops_per_token_head(dk: int, dv: int) -> int:
    # decay (1), S^T k (2), update (2), S^T q (2) multiply-adds per state element
    return 7 * dk * dv
