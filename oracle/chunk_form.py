"""fp64 chunked form of the KDA recurrence — TEST INFRASTRUCTURE ONLY.

Independent statement of the chunk unrolling described in "Kimi K3: the
manos..." section "FlashKDA Algorithm": for a chunk of tokens i..j with
starting state S_in,
    S_j   = D_{j:i} S_in + sum_t D_{j:t+1} k_t u_t^T
    o_j^T = q_j^T D_{j:i} S_in + sum_{t<=j} q_j^T D_{j:t+1} k_t u_t^T
where D_{j:i} is the product of the per-token diagonal decays, and the
pseudo-values u come from the UT transform (I + L) U = Diag(beta)(V - K_decay S_in)
with L strictly lower triangular, L_ts = beta_t k_t^T D_{t:s+1} k_s.

Decay ratios are formed directly as exp(cum_t - cum_s) per channel (the
definition of D_{t:s+1}), not through separate decay / inverse-decay factors,
so the form stays finite for any chunk length. Tests use it only to pin the
chunk algebra against the token-by-token oracle; the GPU path is judged
against the token recurrence.
"""
from __future__ import annotations

import numpy as np


def _chunk(Q, K, V, G, beta, S):
    """One chunk for one head. Q,K,G: [n,dk]; V: [n,dv]; beta: [n]; S: [dk,dv]."""
    n = Q.shape[0]
    cum = np.cumsum(G, axis=0)                      # inclusive: log of D_{t:i}
    t_idx = np.arange(n)[:, None]
    s_idx = np.arange(n)[None, :]
    causal = s_idx <= t_idx
    # log of D_{t:s+1} = cum_t - cum_s for s <= t (zero on the diagonal).
    logr = np.where(causal[:, :, None], cum[:, None, :] - cum[None, :, :], -np.inf)
    R = np.exp(logr)                                # [n, n, dk], zero above the diagonal
    a = np.exp(cum)                                 # diagonal of D_{t:i}
    KK = np.einsum("td,tsd,sd->ts", K, R, K)        # k_t^T D_{t:s+1} k_s
    QK = np.einsum("td,tsd,sd->ts", Q, R, K)        # q_t^T D_{t:s+1} k_s
    L = np.tril(beta[:, None] * KK, -1)             # strictly lower
    Bm = beta[:, None] * (V - (a * K) @ S)
    U = np.linalg.solve(np.eye(n) + L, Bm)          # UT transform
    O = (a * Q) @ S + np.tril(QK) @ U               # causal mask keeps the diagonal
    restore = np.exp(cum[-1][None, :] - cum) * K    # D_{j:t+1} k_t
    S_out = a[-1][:, None] * S + restore.T @ U
    return O, S_out


def chunked_prefill_f64(q, k, v, log_alpha, beta, S0, chunk):
    """Inputs as float64 arrays in the [B,T,H,*] layouts; returns (o, S_final)."""
    q, k, v, la, beta = (np.asarray(x, np.float64) for x in (q, k, v, log_alpha, beta))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, T, H, dv))
    S_fin = np.zeros((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            S = np.zeros((dk, dv)) if S0 is None else np.asarray(S0, np.float64)[b, h].copy()
            for c0 in range(0, T, chunk):
                sl = slice(c0, min(c0 + chunk, T))
                O, S = _chunk(q[b, sl, h], k[b, sl, h], v[b, sl, h], la[b, sl, h],
                              beta[b, sl, h], S)
                o[b, sl, h] = O
            S_fin[b, h] = S
    return o, S_fin
