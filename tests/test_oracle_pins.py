"""Pins of the fp64 oracle to facts fixed outside the oracle itself.

Each test states the passage or the mathematics it follows. None of them
re-types the oracle's two-stage step: they use hand-worked values, closed
forms, the single-matrix product form, the Gated DeltaNet special case,
autograd of the retrieval loss, orthonormal-key retrieval, a chunked
statement of the recurrence and structural properties (linearity,
continuation, tail padding, a norm bound).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle.chunk_form import chunked_prefill_f64

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "kda_hand_example.json")


def rand_inputs(B, T, H, dk, dv, seed, la_hi=0.2, unit=True, s0=True):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    if unit:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    la = -rng.uniform(0.001, la_hi, (B, T, H, dk))
    beta = rng.uniform(0.0, 1.0, (B, T, H))
    S0 = 0.3 * rng.standard_normal((B, H, dk, dv)) if s0 else None
    return q, k, v, la, beta, S0


# ---- hand-worked values (Kimi K3 blog, "Decay Old Memory" / "Apply Delta-Rule Update")

def test_hand_worked_examples():
    cases = json.load(open(GOLDEN))["cases"]
    for c in cases:
        toks = c["tokens"]
        T, dk, dv = len(toks), c["dk"], c["dv"]
        q = np.array([t["q"] for t in toks], float).reshape(1, T, 1, dk)
        k = np.array([t["k"] for t in toks], float).reshape(1, T, 1, dk)
        v = np.array([t["v"] for t in toks], float).reshape(1, T, 1, dv)
        la = np.log(np.array([t["alpha"] for t in toks], float)).reshape(1, T, 1, dk)
        beta = np.array([t["beta"] for t in toks], float).reshape(1, T, 1)
        S0 = np.array(c["S0"], float).reshape(1, 1, dk, dv)
        o, S = oracle.prefill_f64(q, k, v, la, beta, S0)
        want_o = np.array([t["o"] for t in toks], float)
        np.testing.assert_allclose(o[0, :, 0], want_o, rtol=0, atol=1e-14, err_msg=c["name"])
        np.testing.assert_allclose(S[0, 0], np.array(c["S_final"]), rtol=0, atol=1e-14,
                                   err_msg=c["name"])


# ---- closed forms

def test_no_decay_no_write_keeps_state():
    # alpha = 1 and beta = 0: nothing is forgotten, nothing written, so S_t = S0
    # and o_t = S0^T q_t (roles of alpha and beta, Kimi K3 blog).
    q, k, v, la, beta, S0 = rand_inputs(2, 37, 3, 8, 5, 1)
    la[:] = 0.0
    beta[:] = 0.0
    o, S = oracle.prefill_f64(q, k, v, la, beta, S0)
    np.testing.assert_allclose(S, S0, rtol=0, atol=1e-15)
    want = np.stack([np.stack([q[b, :, h] @ S0[b, h] for h in range(3)], 1) for b in range(2)])
    np.testing.assert_allclose(o, want, rtol=0, atol=1e-13)


def test_pure_decay_closed_form():
    # beta = 0: S_t = Diag(prod_{s<=t} alpha_s) S0 (per key channel, i.e. per row).
    q, k, v, la, beta, S0 = rand_inputs(1, 25, 2, 6, 4, 2)
    beta[:] = 0.0
    o, S = oracle.prefill_f64(q, k, v, la, beta, S0)
    cum = np.cumsum(la, axis=1)
    for h in range(2):
        np.testing.assert_allclose(S[0, h], np.exp(cum[0, -1, h])[:, None] * S0[0, h],
                                   rtol=1e-13, atol=0)
        for t in (0, 11, 24):
            St = np.exp(cum[0, t, h])[:, None] * S0[0, h]
            np.testing.assert_allclose(o[0, t, h], St.T @ q[0, t, h], rtol=1e-12, atol=1e-15)


# ---- the single-matrix product form (Kimi K3 blog; trillion-scale page section 4)

def test_product_form_rectangular():
    q, k, v, la, beta, S0 = rand_inputs(1, 40, 2, 7, 3, 3, la_hi=1.0)
    o, S = oracle.prefill_f64(q, k, v, la, beta, S0)
    for h in range(2):
        St = S0[0, h].copy()
        for t in range(40):
            kt = k[0, t, h][:, None]
            A = (np.eye(7) - beta[0, t, h] * kt @ kt.T) @ np.diag(np.exp(la[0, t, h]))
            St = A @ St + beta[0, t, h] * kt @ v[0, t, h][None, :]
            np.testing.assert_allclose(o[0, t, h], St.T @ q[0, t, h], rtol=1e-11, atol=1e-13)
        np.testing.assert_allclose(S[0, h], St, rtol=1e-11, atol=1e-13)


def test_gated_deltanet_scalar_gate():
    # A per-head scalar gate broadcast over the key channels must reproduce
    # Gated DeltaNet: S_t = alpha_t (I - beta_t k k^T) S_{t-1} + beta_t k v^T.
    q, k, v, la, beta, S0 = rand_inputs(1, 30, 1, 6, 6, 4)
    scalar = -np.random.default_rng(9).uniform(0.01, 0.5, 30)
    la[0, :, 0, :] = scalar[:, None]
    o, S = oracle.prefill_f64(q, k, v, la, beta, S0)
    St = S0[0, 0].copy()
    for t in range(30):
        kt = k[0, t, 0][:, None]
        St = math.exp(scalar[t]) * (np.eye(6) - beta[0, t, 0] * kt @ kt.T) @ St \
            + beta[0, t, 0] * kt @ v[0, t, 0][None, :]
    np.testing.assert_allclose(S[0, 0], St, rtol=1e-12, atol=1e-14)


def test_delta_write_is_gradient_step_on_retrieval_loss():
    # "Kimi K3: the manos..." section "DeltaNet": the delta rule minimises the
    # L2 retrieval error. One step of gradient descent with rate beta on
    # 0.5 * ||Sbar^T k - v||^2 from the decayed state must give S_t.
    torch.manual_seed(0)
    dk, dv = 5, 4
    S_prev = torch.randn(dk, dv, dtype=torch.float64)
    k = torch.randn(dk, dtype=torch.float64)
    k = k / k.norm()
    v = torch.randn(dv, dtype=torch.float64)
    q = torch.randn(dk, dtype=torch.float64)
    la = -torch.rand(dk, dtype=torch.float64)
    beta = 0.7
    Sbar = (torch.exp(la)[:, None] * S_prev).requires_grad_(True)
    loss = 0.5 * ((Sbar.T @ k - v) ** 2).sum()
    (grad,) = torch.autograd.grad(loss, Sbar)
    want = (Sbar - beta * grad).detach()
    o, S = oracle.prefill_f64(q.view(1, 1, 1, dk), k.view(1, 1, 1, dk), v.view(1, 1, 1, dv),
                              la.view(1, 1, 1, dk), torch.tensor([[[beta]]], dtype=torch.float64),
                              S_prev.view(1, 1, dk, dv))
    np.testing.assert_allclose(S[0, 0], want.numpy(), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(o[0, 0, 0], (want.T @ q).numpy(), rtol=1e-12, atol=1e-14)


# ---- retrieval facts of the delta rule

def test_full_write_retrieves_last_value_any_decay():
    # beta = 1, ||k|| = 1: S_t^T k_t = v_t whatever alpha; with q_t = k_t, o_t = v_t.
    q, k, v, la, beta, S0 = rand_inputs(1, 50, 2, 16, 8, 5, la_hi=3.0)
    beta[:] = 1.0
    o, _ = oracle.prefill_f64(k, k, v, la, beta, S0)
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-12)


def test_orthonormal_keys_store_every_pair():
    # alpha = 1, beta = 1, S0 = 0, orthonormal keys: S_T = sum_i k_i v_i^T and
    # S_T^T k_i = v_i for every stored pair.
    rng = np.random.default_rng(6)
    d, dv = 12, 5
    Qm, _ = np.linalg.qr(rng.standard_normal((d, d)))
    k = Qm.T.reshape(1, d, 1, d)           # row i = i-th orthonormal key
    v = rng.standard_normal((1, d, 1, dv))
    la = np.zeros((1, d, 1, d))
    beta = np.ones((1, d, 1))
    _, S = oracle.prefill_f64(k, k, v, la, beta, None)
    np.testing.assert_allclose(S[0, 0], k[0, :, 0].T @ v[0, :, 0], atol=1e-13)
    np.testing.assert_allclose(k[0, :, 0] @ S[0, 0], v[0, :, 0], atol=1e-13)


def test_norm_bound():
    # ||(I - beta k k^T) Diag(alpha)||_2 <= 1 for beta ||k||^2 in [0, 2], alpha <= 1,
    # hence ||S_t||_F <= ||S_{t-1}||_F + beta_t ||k_t|| ||v_t||.
    q, k, v, la, beta, S0 = rand_inputs(1, 60, 1, 8, 8, 7, la_hi=0.05)
    prev = np.linalg.norm(S0[0, 0])
    for t in range(60):
        _, S = oracle.prefill_f64(q[:, : t + 1], k[:, : t + 1], v[:, : t + 1],
                                  la[:, : t + 1], beta[:, : t + 1], S0)
        cur = np.linalg.norm(S[0, 0])
        assert cur <= prev + beta[0, t, 0] * np.linalg.norm(v[0, t, 0]) + 1e-12
        prev = cur


# ---- chunked unrolling ("Kimi K3: the manos...", section "FlashKDA Algorithm")

@pytest.mark.parametrize("C", [1, 2, 4, 8, 16, 32, 64])
def test_chunk_form_equals_step_form(C):
    q, k, v, la, beta, S0 = rand_inputs(1, 64, 2, 16, 16, 10 + C)
    o1, S1 = oracle.prefill_f64(q, k, v, la, beta, S0)
    o2, S2 = chunked_prefill_f64(q, k, v, la, beta, S0, C)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(S2, S1, rtol=0, atol=1e-12)


def test_chunk_form_ragged_rectangular():
    q, k, v, la, beta, S0 = rand_inputs(2, 50, 3, 12, 7, 20)
    o1, S1 = oracle.prefill_f64(q, k, v, la, beta, S0)
    o2, S2 = chunked_prefill_f64(q, k, v, la, beta, S0, 16)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(S2, S1, rtol=0, atol=1e-12)


def test_chunk_form_strong_decay():
    # log-decay near the lower end of the (-5, 0) bound ("LLM architecture at
    # trillion scale", section 4): chunk form stays exact in fp64.
    q, k, v, la, beta, S0 = rand_inputs(1, 64, 1, 8, 8, 21)
    la = -np.random.default_rng(3).uniform(3.0, 5.0, la.shape)
    o1, S1 = oracle.prefill_f64(q, k, v, la, beta, S0)
    o2, S2 = chunked_prefill_f64(q, k, v, la, beta, S0, 64)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(S2, S1, rtol=0, atol=1e-12)


# ---- structure

def test_tail_padding_is_exact():
    # Tokens with k = q = v = 0, log alpha = 0, beta = 0 leave the state alone.
    q, k, v, la, beta, S0 = rand_inputs(1, 20, 2, 8, 8, 11)
    o1, S1 = oracle.prefill_f64(q, k, v, la, beta, S0)
    pad = lambda x: np.concatenate([x, np.zeros((1, 12) + x.shape[2:])], axis=1)
    o2, S2 = oracle.prefill_f64(pad(q), pad(k), pad(v), pad(la), pad(beta), S0)
    np.testing.assert_array_equal(S2, S1)
    np.testing.assert_array_equal(o2[:, :20], o1)
    np.testing.assert_array_equal(o2[:, 20:], 0.0)


def test_linear_in_state_and_values():
    q, k, v, la, beta, S0 = rand_inputs(1, 30, 2, 8, 6, 12)
    _, _, v2, _, _, S02 = rand_inputs(1, 30, 2, 8, 6, 13)
    a, b = 0.7, -1.3
    o1, S1 = oracle.prefill_f64(q, k, v, la, beta, S0)
    o2, S2 = oracle.prefill_f64(q, k, v2, la, beta, S02)
    o3, S3 = oracle.prefill_f64(q, k, a * v + b * v2, la, beta, a * S0 + b * S02)
    np.testing.assert_allclose(o3, a * o1 + b * o2, atol=1e-12)
    np.testing.assert_allclose(S3, a * S1 + b * S2, atol=1e-12)


def test_continuation_and_decode_step():
    q, k, v, la, beta, S0 = rand_inputs(2, 33, 2, 8, 8, 14)
    o, S = oracle.prefill_f64(q, k, v, la, beta, S0)
    oa, Sa = oracle.prefill_f64(q[:, :20], k[:, :20], v[:, :20], la[:, :20], beta[:, :20], S0)
    ob, Sb = oracle.prefill_f64(q[:, 20:], k[:, 20:], v[:, 20:], la[:, 20:], beta[:, 20:], Sa)
    np.testing.assert_allclose(np.concatenate([oa, ob], 1), o, atol=1e-13)
    np.testing.assert_allclose(Sb, S, atol=1e-13)
    # a decode step is one token of the recurrence
    od, Sd = oracle.decode_f64(q[:, 0], k[:, 0], v[:, 0], la[:, 0], beta[:, 0], S0)
    o1, S1 = oracle.prefill_f64(q[:, :1], k[:, :1], v[:, :1], la[:, :1], beta[:, :1], S0)
    np.testing.assert_allclose(od, o1[:, 0], atol=1e-15)
    np.testing.assert_allclose(Sd, S1, atol=1e-15)


def test_empty_sequence_returns_initial_state():
    q, k, v, la, beta, S0 = rand_inputs(1, 0, 2, 4, 4, 15)
    o, S = oracle.prefill_f64(q, k, v, la, beta, S0)
    assert o.shape == (1, 0, 2, 4)
    np.testing.assert_array_equal(S, S0)


def test_rel_l2():
    x = np.array([3.0, 4.0])
    assert oracle.rel_l2(x, x) == 0.0
    assert abs(oracle.rel_l2(np.array([3.0, 4.0 + 0.5]), x) - 0.1) < 1e-15


# ---- packed sequences and state checkpoints ("Kimi K3: the manos...",
#      section "KDA Prefix Cache Management": states kept at fixed intervals)

def packed_inputs(lengths, H, dk, dv, seed, la_hi=0.2):
    T = sum(lengths)
    q, k, v, la, beta, _ = rand_inputs(1, T, H, dk, dv, seed, la_hi=la_hi, s0=False)
    S0 = 0.3 * np.random.default_rng(seed + 1).standard_normal((len(lengths), H, dk, dv))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(int).tolist()
    return q[0], k[0], v[0], la[0], beta[0], S0, cu


def test_varlen_orthonormal_keys_closed_form():
    # alpha = 1, beta = 1, S0 = 0, orthonormal keys inside each sequence:
    # the state after j tokens of a sequence is sum_{t<j} k_t v_t^T (each write
    # leaves the earlier, orthogonal keys alone), and o_t = S_t^T q_t.
    rng = np.random.default_rng(30)
    d, dv, K = 12, 5, 3
    lengths = [7, 0, 12, 4]
    T = sum(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(int)
    k = np.zeros((T, 1, d))
    for a, b in zip(cu, cu[1:]):
        Qm, _ = np.linalg.qr(rng.standard_normal((d, d)))
        k[a:b, 0] = Qm.T[: b - a]
    q = rng.standard_normal((T, 1, d))
    v = rng.standard_normal((T, 1, dv))
    o, S, Sc = oracle.prefill_varlen_f64(q, k, v, np.zeros((T, 1, d)), np.ones((T, 1)),
                                         cu.tolist(), None, ckpt_every=K)
    ck = []
    for i, (a, b) in enumerate(zip(cu, cu[1:])):
        run = np.zeros((d, dv))
        for t in range(a, b):
            run = run + np.outer(k[t, 0], v[t, 0])
            np.testing.assert_allclose(o[t, 0], run.T @ q[t, 0], atol=1e-12)
            if (t + 1 - a) % K == 0:
                ck.append(run)
        np.testing.assert_allclose(S[i, 0], run, atol=1e-12)
    assert Sc.shape[0] == sum(n // K for n in lengths) == len(ck)
    np.testing.assert_allclose(Sc[:, 0], np.stack(ck), atol=1e-12)


def test_varlen_pure_decay_closed_form():
    # beta = 0: no writes, S_t = Diag(exp(sum of log-decays)) S0[i] per
    # sequence; checkpoints at every K tokens of the sequence.
    lengths, K = [5, 9, 0, 4], 2
    q, k, v, la, beta, S0, cu = packed_inputs(lengths, 2, 6, 3, 31, la_hi=1.0)
    beta[:] = 0.0
    o, S, Sc = oracle.prefill_varlen_f64(q, k, v, la, beta, cu, S0, ckpt_every=K)
    ck = []
    for i, (a, b) in enumerate(zip(cu, cu[1:])):
        for t in range(a, b):
            St = np.exp(la[a:t + 1].sum(0))[:, :, None] * S0[i]
            np.testing.assert_allclose(o[t], np.einsum("hkv,hk->hv", St, q[t]), atol=1e-13)
            if (t + 1 - a) % K == 0:
                ck.append(St)
        Sb = np.exp(la[a:b].sum(0))[:, :, None] * S0[i]
        np.testing.assert_allclose(S[i], Sb, atol=1e-13)
    np.testing.assert_allclose(Sc, np.stack(ck), atol=1e-13)


def test_varlen_equals_independent_chunk_form():
    # every sequence against the independent NumPy chunk statement from its
    # own S0; checkpoint j = that statement's state after j*K tokens
    lengths, K = [11, 1, 0, 20], 4
    q, k, v, la, beta, S0, cu = packed_inputs(lengths, 2, 8, 5, 32)
    o, S, Sc = oracle.prefill_varlen_f64(q, k, v, la, beta, cu, S0, ckpt_every=K)
    slot = 0
    for i, (a, b) in enumerate(zip(cu, cu[1:])):
        sl = lambda x, n=b: x[None, a:n]
        oc, Scf = chunked_prefill_f64(sl(q), sl(k), sl(v), sl(la), sl(beta), S0[i:i + 1], 8)
        np.testing.assert_allclose(o[a:b], oc[0], atol=1e-12)
        np.testing.assert_allclose(S[i], Scf[0], atol=1e-12)
        for j in range(1, (b - a) // K + 1):
            n = a + j * K
            _, Sj = chunked_prefill_f64(sl(q, n), sl(k, n), sl(v, n), sl(la, n), sl(beta, n),
                                        S0[i:i + 1], 8)
            np.testing.assert_allclose(Sc[slot], Sj[0], atol=1e-12)
            slot += 1
    assert slot == Sc.shape[0]


def test_varlen_sequences_are_independent():
    # changing one sequence's tokens and initial state changes nothing else
    lengths = [6, 9, 5]
    q, k, v, la, beta, S0, cu = packed_inputs(lengths, 2, 4, 4, 33)
    o1, S1, C1 = oracle.prefill_varlen_f64(q, k, v, la, beta, cu, S0, ckpt_every=3)
    v2, S02 = v.copy(), S0.copy()
    v2[6:15] += 1.0
    S02[1] *= -2.0
    o2, S2, C2 = oracle.prefill_varlen_f64(q, k, v2, la, beta, cu, S02, ckpt_every=3)
    np.testing.assert_array_equal(o1[:6], o2[:6])
    np.testing.assert_array_equal(o1[15:], o2[15:])
    np.testing.assert_array_equal(S1[[0, 2]], S2[[0, 2]])
    np.testing.assert_array_equal(C1[[0, 1, 5]], C2[[0, 1, 5]])   # slots of sequences 0 and 2
    assert not np.allclose(o1[6:15], o2[6:15])


# ---- layer prologue and epilogue ("Kimi K3: the manos...", section "Kimi
#      Linear"; the log-decay bound of the trillion-scale page, section 4)

from oracle import layer as OL


def test_l2norm_against_torch_normalize():
    x = np.random.default_rng(40).standard_normal((3, 5, 2, 16)) * 7.0
    ref = torch.nn.functional.normalize(torch.from_numpy(x), dim=-1).numpy()
    np.testing.assert_allclose(OL.l2norm_f64(x, 0.0), ref, rtol=1e-14, atol=1e-15)
    # the eps sits under the square root: a zero row stays zero, a row with
    # squared norm n is divided by sqrt(n + eps)
    z = OL.l2norm_f64(np.zeros((1, 4)), 1e-6)
    np.testing.assert_array_equal(z, 0.0)
    r = OL.l2norm_f64(np.array([[3.0, 4.0]]), 11.0)
    np.testing.assert_allclose(r, [[0.5, 4.0 / 6.0]], rtol=1e-15)


def test_bounded_log_decay_values():
    from scipy.special import expit
    g = np.array([0.0, 10.0, -10.0, 1.5, -40.0])
    la = OL.log_decay_f64(g, OL.GATE_BOUNDED, dk=1, bound=5.0)
    assert la[0] == -2.5                                   # the midpoint of (-5, 0)
    np.testing.assert_allclose(la, -5.0 * expit(g), rtol=1e-15)
    assert np.all(la < 0) and np.all(la > -5.0)            # inside the open interval
    assert np.all(np.diff(OL.log_decay_f64(np.linspace(-8, 8, 50), OL.GATE_BOUNDED, 1)) < 0)
    np.testing.assert_allclose(OL.log_decay_f64(np.array([0.0]), OL.GATE_BOUNDED, 1, bound=3.0),
                               [-1.5])


def test_scalar_gate_is_gated_deltanet():
    # GATE_SCALAR through the layer equals the Gated DeltaNet recurrence
    # S_t = alpha_t (I - beta_t k k^T) S_{t-1} + beta_t k v^T written by hand
    q, k, v, _, beta, S0 = rand_inputs(1, 25, 1, 6, 5, 41)
    a = -np.random.default_rng(42).uniform(0.01, 0.8, (1, 25, 1))
    o, S = OL.layer_prefill_f64(q, k, v, a, beta, S0, gate=OL.GATE_SCALAR)
    St = S0[0, 0].copy()
    for t in range(25):
        kt = k[0, t, 0][:, None]
        St = math.exp(a[0, t, 0]) * (np.eye(6) - beta[0, t, 0] * kt @ kt.T) @ St \
            + beta[0, t, 0] * kt @ v[0, t, 0][None, :]
        np.testing.assert_allclose(o[0, t, 0], St.T @ q[0, t, 0], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(S[0, 0], St, rtol=1e-12, atol=1e-14)


def test_norm_gate_against_torch_rms_norm():
    rng = np.random.default_rng(43)
    o = rng.standard_normal((2, 3, 4, 16)) * 3.0
    z = rng.standard_normal((2, 3, 4, 16))
    w = 1.0 + 0.1 * rng.standard_normal(16)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(o), (16,), torch.from_numpy(w), 1e-6)
    ref = ref.numpy() * torch.sigmoid(torch.from_numpy(z)).numpy()
    np.testing.assert_allclose(OL.norm_gate_f64(o, z, w, 1e-6), ref, rtol=1e-13, atol=1e-14)
    # fully open gate, unit weight: unit RMS per token and head, scale-free
    big = np.full_like(z, 50.0)
    out = OL.norm_gate_f64(o, big, None, 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(out ** 2, axis=-1)), 1.0, rtol=1e-14)
    np.testing.assert_allclose(OL.norm_gate_f64(7.0 * o, big, None, 0.0), out, rtol=1e-13)
    # a closed-half gate (z = 0) halves it
    np.testing.assert_allclose(OL.norm_gate_f64(o, 0 * z, None, 0.0), 0.5 * out, rtol=1e-13)


def test_layer_l2norm_equals_prenormalised_inputs():
    # raw q, k through the layer equal pre-normalised q, k through the op;
    # and scaling raw q, k per token changes nothing
    q, k, v, la, beta, S0 = rand_inputs(1, 20, 2, 8, 6, 44, unit=False)
    tq = torch.nn.functional.normalize(torch.from_numpy(q), dim=-1).numpy()
    tk = torch.nn.functional.normalize(torch.from_numpy(k), dim=-1).numpy()
    o1, S1 = OL.layer_prefill_f64(q, k, v, la, beta, S0, l2norm=True, l2_eps=0.0)
    o2, S2 = oracle.prefill_f64(tq, tk, v, la, beta, S0)
    np.testing.assert_allclose(o1, o2, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(S1, S2, rtol=1e-13, atol=1e-14)
    s = np.random.default_rng(45).uniform(0.5, 9.0, (1, 20, 2, 1))
    o3, _ = OL.layer_prefill_f64(s * q, s * k, v, la, beta, S0, l2norm=True, l2_eps=0.0)
    np.testing.assert_allclose(o3, o1, rtol=1e-12, atol=1e-13)


def test_layer_decode_is_one_layer_prefill_token():
    q, k, v, _, beta, S0 = rand_inputs(2, 1, 3, 8, 8, 46, unit=False)
    g = np.random.default_rng(47).standard_normal((2, 1, 3, 8)) - 3.0
    z = np.random.default_rng(48).standard_normal((2, 1, 3, 8))
    w = np.linspace(0.5, 1.5, 8)
    kw = dict(l2norm=True, gate=OL.GATE_BOUNDED, z=z, w=w)
    o1, S1 = OL.layer_prefill_f64(q, k, v, g, beta, S0, **kw)
    kw["z"] = z[:, 0]
    o2, S2 = OL.layer_decode_f64(q[:, 0], k[:, 0], v[:, 0], g[:, 0], beta[:, 0], S0, **kw)
    np.testing.assert_allclose(o2, o1[:, 0], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(S2, S1, rtol=1e-14, atol=1e-15)
