"""fp64 statement of the KDA layer's weight-free prologue and epilogue —
TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's CPU baseline may import
this module. It imports nothing from the GPU package.

"Kimi K3: the manos...", section "Kimi Linear", describes the operations
around the recurrence. q and k are L2-normalised; the decay comes from a
low-rank projection; the output is normalised per head and scaled by an
output gate. The trillion-scale architecture page, section 4, bounds the
log-decay to (-5, 0). The projections need trained weights and are not here;
these functions take their outputs as inputs:

    q_hat = q / sqrt(sum_d q_d^2 + eps_qk)            (the same for k)
    log_alpha = -bound * sigmoid(g)                   (g: gate pre-activation)
    log_alpha[t, h, :] = a[t, h]                      (scalar per head: Gated DeltaNet)
    out = w * o / sqrt(mean_j o_j^2 + eps_o) * sigmoid(z)   (per token and head, over d_v)

The exact form of the bounding map and of the per-head norm is not printed on
the pages. The readings taken are listed with the design notes: a scaled
sigmoid for the open interval (-bound, 0), and an RMS norm with a weight per
value channel.
"""
from __future__ import annotations

import numpy as np

from . import _f64, decode_f64, prefill_f64

GATE_LOG, GATE_BOUNDED, GATE_SCALAR = 0, 1, 2


def sigmoid(x):
    x = np.asarray(x, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-x))


def l2norm_f64(x, eps):
    """x / sqrt(sum of squares over the last axis + eps)."""
    x = _f64(x)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def log_decay_f64(gate_in, gate, dk, bound=5.0):
    """Per-channel natural log-decay from the gate input of mode `gate`:
    GATE_LOG (given, [..., dk]), GATE_BOUNDED (pre-activation g, [..., dk]:
    -bound * sigmoid(g)) or GATE_SCALAR (one log-decay per token and head,
    [...]: broadcast over the dk key channels)."""
    g = _f64(gate_in)
    if gate == GATE_LOG:
        return g
    if gate == GATE_BOUNDED:
        return -bound * sigmoid(g)
    if gate == GATE_SCALAR:
        return np.repeat(g[..., None], dk, axis=-1)
    raise ValueError(gate)


def norm_gate_f64(o, z, w, eps):
    """w * o / sqrt(mean over d_v of o^2 + eps) * sigmoid(z), per token and head."""
    o, z = _f64(o), _f64(z)
    w = np.ones(o.shape[-1]) if w is None else _f64(w)
    rms = np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    return w * (o / rms) * sigmoid(z)


def _prologue(q, k, gate_in, dk, l2norm, gate, bound, l2_eps):
    if l2norm:
        q, k = l2norm_f64(q, l2_eps), l2norm_f64(k, l2_eps)
    return q, k, log_decay_f64(gate_in, gate, dk, bound)


def layer_prefill_f64(q, k, v, gate_in, beta, S0=None, *, l2norm=False, gate=GATE_LOG,
                      bound=5.0, l2_eps=1e-6, z=None, w=None, out_eps=1e-6, nthreads=None):
    """Prologue, the token recurrence over [B,T,H,*] inputs, then the
    epilogue when z is given. Returns (out [B,T,H,dv], S_final)."""
    dk = q.shape[-1]
    q, k, la = _prologue(q, k, gate_in, dk, l2norm, gate, bound, l2_eps)
    o, S = prefill_f64(q, k, v, la, beta, S0, nthreads=nthreads)
    if z is not None:
        o = norm_gate_f64(o, z, w, out_eps)
    return o, S


def layer_decode_f64(q, k, v, gate_in, beta, S, *, l2norm=False, gate=GATE_LOG, bound=5.0,
                     l2_eps=1e-6, z=None, w=None, out_eps=1e-6, nthreads=None):
    """One decode step with the same prologue and epilogue. Returns (out [B,H,dv], S_new)."""
    dk = q.shape[-1]
    q, k, la = _prologue(q, k, gate_in, dk, l2norm, gate, bound, l2_eps)
    o, S = decode_f64(q, k, v, la, beta, S, nthreads=nthreads)
    if z is not None:
        o = norm_gate_f64(o, z, w, out_eps)
    return o, S
