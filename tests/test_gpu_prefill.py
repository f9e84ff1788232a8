"""GPU parity of kda_prefill_fwd (through the C ABI) against the fp64 oracle.

Small cases are compared element by element over whole tensors; the large
configurations run at full size in the launch configuration the benchmark
times, and are compared on sampled heads the oracle can afford.
"""
import math

import numpy as np
import pytest
import torch

import gated_delta_rule_22_amd as kda
import oracle
import workloads as W
from gpu_helpers import DEV, TOL_BF16, TOL_F32, report, to_dev

pytestmark = pytest.mark.gpu


def gpu_prefill(xd, chunk=64, S0="x", **kw):
    s0 = xd["S0"] if isinstance(S0, str) else S0
    o, S = kda.kda_prefill_fwd(xd["q"], xd["k"], xd["v"], xd["log_alpha"], xd["beta"], s0,
                               chunk=chunk, **kw)
    torch.cuda.synchronize()
    return o, S


def oracle_prefill(x, S0="x"):
    s0 = x["S0"] if isinstance(S0, str) else S0
    return oracle.prefill_f64(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], s0)


def test_cpu_sized_config_fp32():
    c = W.PREFILL_CONFIGS["cpu"]
    x = W.prefill_inputs(c)
    o, S = gpu_prefill(to_dev(x), chunk=c.chunk)
    ro, rS = oracle_prefill(x)
    report("cpu config fp32 B1 H2 T64 D16 C16", [("o", o, ro), ("S", S, rS)], TOL_F32)


@pytest.mark.parametrize("dk,dv,T,chunk", [(16, 16, 64, 16), (32, 64, 100, 32),
                                           (64, 32, 77, 64), (128, 128, 40, 64),
                                           (16, 128, 130, 16), (128, 16, 33, 32)])
def test_fp32_shapes_ragged(dk, dv, T, chunk):
    c = W.PREFILL_CONFIGS["batched"]
    import dataclasses
    c = dataclasses.replace(c, dk=dk, dv=dv)
    x = W.prefill_inputs(c, B=2, T=T, H=3, dtype=torch.float32)
    o, S = gpu_prefill(to_dev(x), chunk=chunk)
    ro, rS = oracle_prefill(x)
    report(f"fp32 dk{dk} dv{dv} T{T} C{chunk}", [("o", o, ro), ("S", S, rS)], TOL_F32)


@pytest.mark.parametrize("base,B,H,T", [("prefill", 1, 16, 4096), ("batched", 2, 8, 2000)])
def test_fp32_at_config_size(base, B, H, T):
    """fp32 inputs at the 4K configuration's full size (and a ragged batch
    with the batched configuration's carried state and decay mix): 64 chunks
    of fp32 state carry on the generic kernel, every head, against the
    fp32 bar."""
    c = W.PREFILL_CONFIGS[base]
    x = W.prefill_inputs(c, B=B, T=T, H=H, dtype=torch.float32)
    o, S = gpu_prefill(to_dev(x))
    ro, rS = oracle_prefill(x)
    report(f"fp32 {base} B{B} H{H} T{T}", [("o", o, ro), ("S", S, rS)], TOL_F32)


@pytest.mark.parametrize("T", [1, 17, 64, 200, 256])
def test_bf16_mfma_small(T):
    c = W.PREFILL_CONFIGS["batched"]
    x = W.prefill_inputs(c, B=2, T=T, H=3)
    o, S = gpu_prefill(to_dev(x))
    ro, rS = oracle_prefill(x)
    report(f"bf16 B2 H3 T{T} D128 C64 with S0", [("o", o, ro), ("S", S, rS)], TOL_BF16)


def test_bf16_fused_half_width_path():
    # 128..255 heads: the fused kernel with 64-column workgroups
    c = W.PREFILL_CONFIGS["batched"]
    x = W.prefill_inputs(c, B=2, T=130, H=64)
    o, S = gpu_prefill(to_dev(x))
    ro, rS = oracle_prefill(x)
    report("bf16 B2 H64 T130 (fused, 64-column blocks)", [("o", o, ro), ("S", S, rS)], TOL_BF16)


@pytest.mark.parametrize("with_s0", [False, True])
def test_bf16_fused_full_width_path(with_s0):
    # 256+ heads: the fused kernel with one 128-column workgroup per head
    c = W.PREFILL_CONFIGS["batched"]
    x = W.prefill_inputs(c, B=4, T=130, H=64)
    if not with_s0:
        x["S0"] = None
    o, S = gpu_prefill(to_dev(x))
    ro, rS = oracle_prefill(x)
    report(f"bf16 B4 H64 T130 (fused, 128-column blocks, S0={with_s0})",
           [("o", o, ro), ("S", S, rS)], TOL_BF16)


def test_bf16_workspace_given_by_caller():
    # few heads use the chunk-parallel prep + state kernels through a workspace
    c = W.PREFILL_CONFIGS["prefill"]
    x = W.prefill_inputs(c, B=1, T=333, H=5)
    xd = to_dev(x)
    n = kda.kda_prefill_workspace_size(1, 333, 5, 128, 128, torch.bfloat16)
    assert n > 0
    ws = torch.full((n,), 0x7f, dtype=torch.uint8, device=DEV)
    o, S = gpu_prefill(xd, workspace=ws)
    ro, rS = oracle_prefill(x)
    report("bf16 B1 H5 T333 with caller workspace", [("o", o, ro), ("S", S, rS)], TOL_BF16)


def test_bf16_prefill_config_full():
    c = W.PREFILL_CONFIGS["prefill"]
    x = W.prefill_inputs(c)
    o, S = gpu_prefill(to_dev(x))
    ro, rS = oracle_prefill(x)
    report("prefill config B1 H16 T4096 D128 (all heads)", [("o", o, ro), ("S", S, rS)], TOL_BF16)


def test_bf16_batched_config_full():
    # every one of the 256 sequence-heads (about 2.1M token-heads for the
    # oracle, a few seconds on the host's cores)
    c = W.PREFILL_CONFIGS["batched"]
    xd = W.prefill_inputs(c, device=DEV)
    o, S = gpu_prefill(xd)
    x = {n: (t.cpu() if t is not None else None) for n, t in xd.items()}
    del xd
    ro, rS = oracle_prefill(x)
    report("batched config B8 H32 T8192 (all heads)", [("o", o, ro), ("S", S, rS)], TOL_BF16)


@pytest.fixture(scope="module")
def long_case():
    """The 1M-token configuration at full size, built head by head from the
    per-head seeds, and one prefill call on it (the benchmark's launch
    configuration)."""
    c = W.PREFILL_CONFIGS["long"]
    x = W.prefill_inputs_by_head(c, device=DEV)
    o, S = kda.kda_prefill_fwd(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], None)
    torch.cuda.synchronize()
    yield dict(q=x["q"], k=x["k"], v=x["v"], la=x["log_alpha"], beta=x["beta"], o=o, S=S,
               T=c.T)
    del x, o, S
    torch.cuda.empty_cache()


def _window_from_zero(x, heads, a, Wn):
    """Oracle outputs of the given heads on tokens [a, a + Wn) from a zero
    state, and the damping bound of the history: over those heads, the
    largest product of the largest per-step decay over the first half of the
    window (outputs are compared only in the second half, where the true
    history is damped by at least that) and over the whole window (for the
    final state)."""
    win = slice(a, a + Wn)
    part = lambda t: t[:, win][:, :, heads].cpu()
    lmax = x["la"][0, win][:, heads].double().max(dim=-1).values      # [Wn, heads]
    damp_o = float(torch.exp(lmax[:Wn // 2].sum(dim=0)).max())
    damp_s = float(torch.exp(lmax.sum(dim=0)).max())
    ro, rS = oracle.prefill_f64(part(x["q"]), part(x["k"]), part(x["v"]), part(x["la"]),
                                part(x["beta"]), None)
    return ro, rS, damp_o, damp_s


def test_bf16_long_config_sampled(long_case):
    """1M-token context at full size, every head. The first 65536 tokens are
    checked exactly; the end against a run of the last 65536 tokens from a
    zero state: the state entering that window is damped by the product of
    the largest per-step decay over the window, which the test computes for
    every head and requires to be negligible against the tolerance (outputs
    are compared only in the second half of the window, where the same
    holds)."""
    x = long_case
    T, o, S = x["T"], x["o"], x["S"]
    H = o.shape[2]
    Wn = 65536
    skip = Wn // 2
    heads = list(range(H))
    first = slice(0, Wn)
    part = lambda t: t[:, first].cpu()
    ro, _ = oracle.prefill_f64(part(x["q"]), part(x["k"]), part(x["v"]), part(x["la"]),
                               part(x["beta"]), None)
    report(f"long config first {Wn} tokens, all {H} heads", [("o", o[:, first], ro)], TOL_BF16)
    del ro
    ro, rS, damp_o, damp_s = _window_from_zero(x, heads, T - Wn, Wn)
    assert damp_o < 1e-6 and damp_s < 1e-6, (damp_o, damp_s)
    report(f"long config last {Wn - skip} tokens + final state, all {H} heads "
           f"(damping {damp_o:.1e} / {damp_s:.1e})",
           [("o", o[:, T - Wn + skip:], ro[:, skip:]), ("S", S, rS)], TOL_BF16)


def test_bf16_long_config_mid_window(long_case):
    """The same 1M-token call, a window in the middle of the sequence (tokens
    524,288 .. 589,824) on four heads, against the oracle run from a zero
    state at the window start, under the same damping bound."""
    x = long_case
    heads, a, Wn = [3, 11, 19, 27], x["T"] // 2, 65536
    skip = Wn // 2
    ro, _, damp_o, _ = _window_from_zero(x, heads, a, Wn)
    assert damp_o < 1e-6, damp_o
    report(f"long config tokens {a + skip}..{a + Wn}, heads {heads} (damping {damp_o:.1e})",
           [("o", x["o"][:, a + skip:a + Wn][:, :, heads], ro[:, skip:])], TOL_BF16)


def test_split_path_regimes_alternate_within_workgroup():
    # Few heads with enough chunks that each prep workgroup takes several in
    # a row (B1 H2 T32768: 4 chunks per workgroup), with a strongly decaying
    # channel in every other chunk: the workgroup alternates between the
    # chunk-level decay reference and the 16-token block factorisation.
    c = W.PREFILL_CONFIGS["prefill"]
    T = 32768
    x = W.prefill_inputs(c, B=1, T=T, H=2)
    for ch in range(1, T // 64, 2):
        x["log_alpha"][:, ch * 64 + 8:ch * 64 + 16, :, (3 * ch) % 128] = -1.5   # e^-12 over 8 tokens
    o, S = gpu_prefill(to_dev(x))
    ro, rS = oracle_prefill(x)
    report("split path, regimes alternating per chunk, B1 H2 T32768",
           [("o", o, ro), ("S", S, rS)], TOL_BF16)


def test_piecewise_split_path_all_heads():
    # Few heads with records that would outgrow the last-level cache: the
    # split path runs prep and state walk piece by piece along the sequence
    # (about 3072 chunk-heads per piece; B1 H4 T65536: pieces of 768 and 256
    # chunks), the state carried in S_final. The workspace holds one piece.
    c = W.PREFILL_CONFIGS["long"]
    x = W.prefill_inputs(c, B=1, T=65536, H=4, seed=31)
    piece = 4 * 768 * 72192 + 4 * 128 * 128 * 4          # records + carried state
    assert kda.kda_prefill_workspace_size(1, 65536, 4, 128, 128, torch.bfloat16) == piece
    o, S = gpu_prefill(to_dev(x))
    ro, rS = oracle_prefill(x)
    report("piecewise split path B1 H4 T65536", [("o", o, ro), ("S", S, rS)], TOL_BF16)


def test_piecewise_split_path_many_heads():
    # 100 sequence-heads (below the fused path's 128): the piece is
    # 3072 / 100 = 30 chunks, so B1 H100 T2560 (40 chunks, 289 MB of records)
    # runs a piece of 30 and a last one of 10, all heads checked
    c = W.PREFILL_CONFIGS["batched"]
    x = W.prefill_inputs(c, B=1, T=2560, H=100, seed=33)
    piece = 100 * 30 * 72192 + 100 * 128 * 128 * 4
    assert kda.kda_prefill_workspace_size(1, 2560, 100, 128, 128, torch.bfloat16) == piece
    o, S = gpu_prefill(to_dev(x))
    ro, rS = oracle_prefill(x)
    report("piecewise split path B1 H100 T2560", [("o", o, ro), ("S", S, rS)], TOL_BF16)


@pytest.mark.parametrize("B,H,T", [(1, 48, 333), (3, 20, 200)])
def test_split_path_32_column_walk(B, H, T):
    # 33 to 127 sequence-heads: the state walk takes 32 value columns per
    # workgroup (four per sequence-head), one round of workgroups
    c = W.PREFILL_CONFIGS["batched"]
    x = W.prefill_inputs(c, B=B, T=T, H=H, seed=41)
    o, S = gpu_prefill(to_dev(x))
    ro, rS = oracle_prefill(x)
    report(f"split path, 32-column walk B{B} H{H} T{T}", [("o", o, ro), ("S", S, rS)], TOL_BF16)


@pytest.mark.parametrize("mode", ["S_final", "no_state", "in_place"])
def test_piecewise_split_path_batch_ragged(mode):
    # Two sequences (strided windows of the batch), a carried S0 and a ragged
    # last piece ending in a chunk of 33 tokens (801 chunks per sequence:
    # pieces of 768 and 33); the state carried in S_final, in the workspace
    # (no S_final wanted), or in S0 itself (S_final = S0).
    c = W.PREFILL_CONFIGS["batched"]
    T = 800 * 64 + 33
    x = W.prefill_inputs(c, B=2, T=T, H=2, seed=32)
    xd = to_dev(x)
    if mode == "S_final":
        o, S = gpu_prefill(xd)
    elif mode == "no_state":
        o, S = gpu_prefill(xd, want_state=False)
        assert S is None
    else:
        S_io = xd["S0"].clone()
        o, S = gpu_prefill(xd, S0=S_io, S_final=S_io)
    ro, rS = oracle_prefill(x)
    pairs = [("o", o, ro)] + ([("S", S, rS)] if S is not None else [])
    report(f"piecewise split path B2 H2 T{T} ({mode})", pairs, TOL_BF16)


@pytest.mark.parametrize("B,H", [(1, 2), (2, 64), (4, 64)])   # split, fused 64- and 128-column
def test_decay_past_the_bound_stays_finite(B, H):
    # Log-decays of -8 to -20 per step, outside the supported [-5, 0]: on
    # one channel over whole 16-token blocks, and on every channel for a few
    # tokens. The matrix-core path clamps them to -5 (keeping exp(-5) of the
    # old state instead of less), so its results stay finite and within the
    # bf16 tolerance of the exact recurrence.
    c = W.PREFILL_CONFIGS["prefill"]
    x = W.prefill_inputs(c, B=B, T=200, H=H)
    g = torch.Generator().manual_seed(5)
    deep = lambda shape: -8.0 - 12.0 * torch.rand(shape, generator=g)
    x["log_alpha"][:, 16:48, :, 9] = deep(x["log_alpha"][:, 16:48, :, 9].shape)
    x["log_alpha"][:, 130:134] = deep(x["log_alpha"][:, 130:134].shape)
    o, S = gpu_prefill(to_dev(x))
    assert torch.isfinite(o.float()).all() and torch.isfinite(S).all()
    if B * H > 8:   # oracle on a few heads
        idx = [0, H // 2, H - 1]
        x = {k: (None if v is None else v[:1, :, idx] if k != "S0" else v[:1, idx])
             for k, v in x.items()}
        o, S = o[:1, :, idx], S[:1, idx]
    ro, rS = oracle_prefill(x)
    report(f"log-decay -8..-20 B{B} H{H} T200", [("o", o, ro), ("S", S, rS)], TOL_BF16)


@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_chunk_size_changes_nothing(chunk):
    c = W.PREFILL_CONFIGS["prefill"]
    x = W.prefill_inputs(c, B=1, T=150, H=2)
    o, S = gpu_prefill(to_dev(x), chunk=chunk)
    ro, rS = oracle_prefill(x)
    report(f"bf16 chunk {chunk} T150", [("o", o, ro), ("S", S, rS)], TOL_BF16)


def test_split_sequence_continuation():
    c = W.PREFILL_CONFIGS["batched"]
    x = W.prefill_inputs(c, B=1, T=320, H=4)
    xd = to_dev(x)
    cut = lambda d, sl: {n: (t[:, sl] if n != "S0" else t) for n, t in d.items()}
    oa, Sa = gpu_prefill(cut(xd, slice(0, 128)))
    ob, Sb = gpu_prefill(cut(xd, slice(128, 320)), S0=Sa)
    o, S = gpu_prefill(xd)
    ro, rS = oracle_prefill(x)
    report("split 128+192 vs oracle", [("o", torch.cat([oa, ob], 1), ro), ("S", Sb, rS)], TOL_BF16)
    report("split vs one shot", [("S", Sb, S.cpu().double().numpy())], 5e-3)


@pytest.mark.parametrize("B,H", [(1, 2), (2, 64), (4, 64)])   # split, fused 64- and 128-column
def test_state_in_place(B, H):
    c = W.PREFILL_CONFIGS["batched"]
    x = W.prefill_inputs(c, B=B, T=130, H=H)
    xd = to_dev(x)
    S = xd["S0"].clone()
    o, Sf = gpu_prefill(xd, S0=S, S_final=S)
    assert Sf.data_ptr() == S.data_ptr()
    ro, rS = oracle_prefill(x)
    report(f"in-place S_final = S0, B{B} H{H}", [("o", o, ro), ("S", S, rS)], TOL_BF16)


def test_empty_sequence_copies_state():
    c = W.PREFILL_CONFIGS["batched"]
    x = W.prefill_inputs(c, B=2, T=0, H=3)
    xd = to_dev(x)
    o, S = gpu_prefill(xd)
    assert o.shape == (2, 0, 3, 128)
    assert torch.equal(S, xd["S0"])
    o, S = gpu_prefill(xd, S0=None)
    assert torch.count_nonzero(S) == 0


def test_no_decay_no_write_keeps_state_exactly():
    c = W.PREFILL_CONFIGS["batched"]
    x = W.prefill_inputs(c, B=1, T=190, H=2)
    x["beta"].zero_()
    x["log_alpha"].zero_()
    xd = to_dev(x)
    o, S = gpu_prefill(xd)
    assert torch.equal(S, xd["S0"])
    ro, _ = oracle_prefill(x)
    report("beta=0, alpha=1: o = S0^T q", [("o", o, ro)], TOL_BF16)


def test_strong_decay_at_bound():
    # log-decay in [-5, -4]: the lower end of the supported range
    c = W.PREFILL_CONFIGS["batched"]
    x = W.prefill_inputs(c, B=1, T=192, H=2)
    x["log_alpha"] = -4.0 - torch.rand(x["log_alpha"].shape, generator=torch.Generator().manual_seed(1))
    o, S = gpu_prefill(to_dev(x))
    assert torch.isfinite(o.float()).all() and torch.isfinite(S).all()
    ro, rS = oracle_prefill(x)
    report("log-decay in [-5,-4]", [("o", o, ro), ("S", S, rS)], TOL_BF16)


@pytest.mark.parametrize("B,H", [(1, 2), (2, 64), (4, 64)])
def test_decay_regime_changes_between_chunks(B, H):
    # Mild decay, except one channel that drops by e^-12 over tokens 72-79
    # (chunk 1) and by e^-16 over tokens 192-199 (the ragged last chunk):
    # those chunks take the 16-token block factorisation, the others the
    # chunk-level decay reference. Few heads (prep + state kernels) and
    # many heads (both fused variants).
    c = W.PREFILL_CONFIGS["prefill"]
    x = W.prefill_inputs(c, B=B, T=200, H=H)
    x["log_alpha"][:, 72:80, :, 5] = -1.5
    x["log_alpha"][:, 192:200, :, 7] = -2.0
    o, S = gpu_prefill(to_dev(x))
    if B * H > 8:   # oracle on a few heads
        idx = [0, H // 2, H - 1]
        x = {k: (None if v is None else v[:1, :, idx]) for k, v in x.items()}
        o, S = o[:1, :, idx], S[:1, idx]
    ro, rS = oracle_prefill(x)
    report(f"decay regimes B{B} H{H} T200", [("o", o, ro), ("S", S, rS)], TOL_BF16)


def test_basis_keys_store_and_retrieve():
    # alpha = 1, beta = 1, S0 = 0, keys are signed basis vectors (exact in bf16):
    # the final state maps every key back to its value.
    T, D = 128, 128
    g = torch.Generator().manual_seed(3)
    perm = torch.randperm(D, generator=g)
    sign = torch.where(torch.rand(D, generator=g) < 0.5, -1.0, 1.0)
    keys = torch.zeros(T, D)
    keys[torch.arange(T), perm] = sign
    vals = torch.randn(T, D, generator=g)
    x = dict(q=keys.view(1, T, 1, D).bfloat16(), k=keys.view(1, T, 1, D).bfloat16(),
             v=vals.view(1, T, 1, D).bfloat16(), log_alpha=torch.zeros(1, T, 1, D),
             beta=torch.ones(1, T, 1), S0=None)
    o, S = gpu_prefill(to_dev(x))
    retrieved = keys @ S[0, 0].cpu()
    report("basis keys: k_i^T S = v_i", [("retrieved", retrieved, x["v"][0, :, 0].double().numpy())],
           TOL_BF16)
    ro, rS = oracle_prefill(x)
    report("basis keys vs oracle", [("o", o, ro), ("S", S, rS)], TOL_BF16)


def test_prefill_of_one_token_is_a_decode_step():
    c = W.PREFILL_CONFIGS["batched"]
    x = W.prefill_inputs(c, B=2, T=1, H=4)
    xd = to_dev(x)
    o, S = gpu_prefill(xd)
    Sd = xd["S0"].clone()
    od = kda.kda_decode_step(xd["q"][:, 0].contiguous(), xd["k"][:, 0].contiguous(),
                             xd["v"][:, 0].contiguous(), xd["log_alpha"][:, 0].contiguous(),
                             xd["beta"][:, 0].contiguous(), Sd)
    torch.cuda.synchronize()
    report("T=1 prefill vs decode", [("o", o[:, 0], od.cpu().double().numpy()),
                                     ("S", S, Sd.cpu().double().numpy())], TOL_BF16)


def test_deterministic():
    c = W.PREFILL_CONFIGS["batched"]
    xd = to_dev(W.prefill_inputs(c, B=2, T=300, H=4))
    o1, S1 = gpu_prefill(xd)
    o2, S2 = gpu_prefill(xd)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


@pytest.mark.parametrize("H", [4, 64])   # prep + state walk; fused
def test_prefill_then_decode_equals_prefill_of_concatenation(H):
    # serving's hand-over: prefill a prompt, then decode token by token from
    # its final state; the same tokens prefilled in one call must agree
    c = W.PREFILL_CONFIGS["batched"]
    B, T, m = 4, 150, 6
    x = W.prefill_inputs(c, B=B, T=T + m, H=H)
    xd = to_dev(x)
    head = {n: (v[:, :T].contiguous() if n != "S0" else v) for n, v in xd.items()}
    _, S = gpu_prefill(head)
    outs = []
    for t in range(T, T + m):
        step = {n: xd[n][:, t].contiguous() for n in ("q", "k", "v", "log_alpha", "beta")}
        outs.append(kda.kda_decode_step(step["q"], step["k"], step["v"], step["log_alpha"],
                                        step["beta"], S))
    torch.cuda.synchronize()
    o_all, S_all = gpu_prefill(xd)
    o_dec = torch.stack(outs, dim=1)
    report(f"prefill T{T} + {m} decode steps vs prefill T{T + m}, H{H}",
           [("o", o_dec, o_all[:, T:].cpu().double().numpy()),
            ("S", S, S_all.cpu().double().numpy())], TOL_BF16)
    ro, rS = oracle_prefill(x)
    report(f"prefill + decode vs oracle, H{H}", [("o", o_dec, ro[:, T:]), ("S", S, rS)], TOL_BF16)


@pytest.mark.parametrize("H", [65536, 65537])
def test_head_count_limit(H):
    """The matrix-core prefill takes up to 65536 heads per token row: its
    chunk loads address one chunk of every head through 32-bit buffer
    offsets, and at 65536 heads the 64 log-decay rows of a chunk span just
    under 2^31 bytes. One head more takes the generic bf16 kernel. Both at
    one full chunk plus a one-token chunk (the largest offsets of the first
    chunk, then a ragged tail), checked on sampled heads, the last included."""
    c = W.PREFILL_CONFIGS["prefill"]
    xd = W.prefill_inputs(c, B=1, T=65, H=H, seed=65, device=DEV)
    o, S = gpu_prefill(xd, S0=None)
    heads = [0, 1, H // 2, H - 2, H - 1]
    x = {n: (t[:, :, heads].cpu() if t is not None else None) for n, t in xd.items()}
    ro, rS = oracle_prefill(x, S0=None)
    report(f"head-count limit B1 T65 H{H}, heads {heads}",
           [("o", o[:, :, heads], ro), ("S", S[:, heads], rS)], TOL_BF16)
    del xd, o, S
    torch.cuda.empty_cache()
