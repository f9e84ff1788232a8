"""GPU parity of kda_prefill_varlen (packed sequences, state checkpoints)
through the C ABI against the fp64 oracle.

Covers the three bf16 paths (fused with 128- and 64-column workgroups, the
prep + state-walk split for few sequence-heads) and the fp32 path. The length
mixes include empty, one-token, chunk-boundary and ragged sequences, and
checkpoints at several intervals. Further cases: equality with the
fixed-length entry point, offsets that are out of order or out of range,
and too few checkpoint slots.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_22_amd as kda
import oracle
import workloads as W
from gpu_helpers import per_head_rel_l2, DEV, TOL_BF16, TOL_F32, report, to_dev

pytestmark = pytest.mark.gpu


def run_gpu(x, ckpt_every=0, chunk=64, **kw):
    xd = to_dev(x)
    o, S, Sc = kda.kda_prefill_varlen(xd["q"], xd["k"], xd["v"], xd["log_alpha"], xd["beta"],
                                      xd["cu_seqlens"], xd["S0"], ckpt_every=ckpt_every,
                                      chunk=chunk, **kw)
    torch.cuda.synchronize()
    return o, S, Sc


def run_oracle(x, ckpt_every=0, cu=None):
    return oracle.prefill_varlen_f64(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"],
                                     x["cu_seqlens"] if cu is None else cu, x["S0"],
                                     ckpt_every=ckpt_every)


def check(label, x, got, ref, tol):
    o, S, Sc = got
    ro, rS, rSc = ref
    pairs = [("o", o, ro), ("S_final", S, rS)]
    if rSc.shape[0]:
        assert Sc is not None and Sc.shape[0] >= rSc.shape[0]
        pairs.append(("S_ckpt", Sc[:rSc.shape[0]], rSc))
    report(label, pairs, tol)
    # every sequence on its own as well (a wrong offset hides in a global norm)
    cu = x["cu_seqlens"].tolist()
    for i in range(len(cu) - 1):
        a, b = cu[i], cu[i + 1]
        if b > a:
            e = oracle.rel_l2(o[a:b].cpu(), ro[a:b])
            assert e <= tol, f"{label}: sequence {i} o rel-L2 {e:.3e}"
            e, h = per_head_rel_l2(o[a:b].cpu(), ro[a:b], (1,))
            assert e <= tol, f"{label}: sequence {i} head {h} o rel-L2 {e:.3e}"
        e = oracle.rel_l2(S[i].cpu(), rS[i])
        assert e <= tol, f"{label}: sequence {i} S_final rel-L2 {e:.3e}"


BASE = W.PREFILL_CONFIGS["batched"]


@pytest.mark.parametrize("lengths,H,ckpt", [
    ([64, 0, 1, 63, 65, 130, 512, 200, 128, 7, 0, 300, 256, 64, 1, 90], 16, 64),   # fused, 128 cols
    ([700, 1, 0, 129, 512, 33, 64, 260], 24, 128),                               # fused, 64 cols
    ([1000, 0, 2500, 513], 4, 512),                                              # prep + state walk
    ([900, 1, 0, 300, 129, 64, 65], 12, 64),                    # prep + 32-column state walk
    ([3000], 2, 256),                                                            # one sequence, split
    ([0, 0, 90], 3, 64),                                                         # leading empties
])
def test_bf16_paths(lengths, H, ckpt):
    x = W.varlen_inputs(BASE, lengths, H=H, seed=21)
    got = run_gpu(x, ckpt_every=ckpt)
    check(f"bf16 varlen N{len(lengths)} H{H} T{sum(lengths)} ckpt {ckpt}", x, got,
          run_oracle(x, ckpt), TOL_BF16)


# The split schedule (N * H >= 256): a sequence longer than its share of an
# evenly spread call, M = ceil(total chunks * H / 256) chunks, runs its first
# m chunks in the fused kernel (m = M rounded down to whole checkpoint
# intervals) and the rest in the prep + state walk, from the fused part's
# end state. split_slots() reads back which sequences the device split.
def split_slots(ws, N):
    """mslot of the split schedule's tables in a varlen workspace: the tables
    follow the 256-aligned sequence table of 3N + 3 ints as ord, lens1, mslot
    [N] (the library's workspace layout for this schedule)."""
    sp = ((3 * N + 3) * 4 + 255) & ~255
    ints = ws[sp:sp + 12 * N].cpu().view(torch.int32)
    return ints[2 * N:3 * N].tolist()


@pytest.mark.parametrize("lengths,H,ckpt,split", [
    ([64, 2048, 64, 64, 1, 64, 64, 64], 32, 0, [1]),              # m = 5 chunks
    ([64, 2048, 64, 64, 1, 64, 64, 64], 32, 512, [1]),            # m = 8: one checkpoint each side
    ([3000, 100, 0, 65, 2500] + [64] * 11, 16, 128, [0, 4]),      # two split, ragged ends
    ([3000, 64, 500, 64], 128, 256, [0]),                          # room for one split sequence
    ([5000, 64, 4000, 64, 3000, 64], 64, 512, [0, 2]),            # 47 chunks: under the share of 48
])
def test_bf16_split_schedule(lengths, H, ckpt, split):
    x = W.varlen_inputs(BASE, lengths, H=H, seed=31)
    N, T = len(lengths), sum(lengths)
    nbytes = kda.kda_prefill_varlen_workspace_size(N, T, H, 128, 128, torch.bfloat16)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    got = run_gpu(x, ckpt_every=ckpt, workspace=ws)
    slots = split_slots(ws, N)
    assert [i for i in range(N) if slots[i] >= 0] == split, slots
    check(f"bf16 varlen split schedule N{N} H{H} T{T} ckpt {ckpt}", x, got,
          run_oracle(x, ckpt), TOL_BF16)


def test_bf16_split_schedule_without_final_state():
    # no S_final: the first segment's end state still reaches the walk
    lengths = [64, 2048, 64, 64, 1, 64, 64, 64]
    x = W.varlen_inputs(BASE, lengths, H=32, seed=32)
    o, S, _ = run_gpu(x, want_state=False)
    assert S is None
    ro, _, _ = run_oracle(x)
    report("bf16 varlen split schedule, no S_final", [("o", o, ro, (1,))], TOL_BF16)


def test_bf16_split_schedule_in_place():
    # S_final = S0: the walk writes each split sequence's final state over
    # its S0 row, which the fused kernel read in the launch before
    lengths = [3000, 100, 0, 65, 2500] + [64] * 11
    x = W.varlen_inputs(BASE, lengths, H=16, seed=34)
    xd = to_dev(x)
    S_io = xd["S0"].clone()
    o, S, _ = kda.kda_prefill_varlen(xd["q"], xd["k"], xd["v"], xd["log_alpha"], xd["beta"],
                                     xd["cu_seqlens"], S_io, S_final=S_io)
    torch.cuda.synchronize()
    assert S.data_ptr() == S_io.data_ptr()
    ro, rS, _ = run_oracle(x)
    report("bf16 varlen split schedule, S_final = S0", [("o", o, ro, (1,)), ("S_final", S, rS)],
           TOL_BF16)


def test_bf16_split_schedule_many_entries():
    # H = 1, 300 sequences: the 100 of 16 chunks exceed the even share (M = 8)
    # and are all split, so the second table has 100 entries (the prep's
    # chunk map reads entries 64-99 from its second lane-distributed half)
    lengths = [64, 1024, 64] * 100
    x = W.varlen_inputs(BASE, lengths, H=1, seed=35)
    N, T = len(lengths), sum(lengths)
    nbytes = kda.kda_prefill_varlen_workspace_size(N, T, 1, 128, 128, torch.bfloat16)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    got = run_gpu(x, ckpt_every=256, workspace=ws)
    slots = split_slots(ws, N)
    assert sorted(s for s in slots if s >= 0) == list(range(100))
    assert [i for i in range(N) if slots[i] >= 0] == list(range(1, N, 3))
    check(f"bf16 varlen split schedule, 100 split of {N}, H1", x, got, run_oracle(x, 256),
          TOL_BF16)


def test_bf16_split_schedule_chunk_budget():
    # second segments are capped at 16384 / H chunks (256 at H = 64): the
    # 30,000-token sequence (469 chunks, M = 118) keeps 213 in the fused
    # kernel instead of 118. Inputs on the device; the oracle checks two
    # heads of the long sequence and every head of the short ones.
    lengths, H = [64, 64, 30000, 64], 64
    x = W.varlen_inputs(BASE, lengths, H=H, seed=33, device=DEV)
    N, T = len(lengths), sum(lengths)
    nbytes = kda.kda_prefill_varlen_workspace_size(N, T, H, 128, 128, torch.bfloat16)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    xd = dict(x)
    xd["cu_seqlens"] = x["cu_seqlens"].to(DEV)
    o, S, _ = kda.kda_prefill_varlen(xd["q"], xd["k"], xd["v"], xd["log_alpha"], xd["beta"],
                                     xd["cu_seqlens"], xd["S0"], workspace=ws)
    torch.cuda.synchronize()
    sp = ((3 * N + 3) * 4 + 255) & ~255
    ints = ws[sp:sp + 12 * N].cpu().view(torch.int32).tolist()
    assert ints[N:2 * N] == [64, 64, 213 * 64, 64]          # fused lengths
    assert ints[2 * N:3 * N] == [-1, -1, 0, -1]              # the long one is split
    cu = x["cu_seqlens"].tolist()
    for i, heads in ((2, [5, 42]), (0, list(range(H))), (3, list(range(H)))):
        a, b = cu[i], cu[i + 1]
        sub = {n: x[n][a:b][:, heads].cpu() for n in ("q", "k", "v", "log_alpha", "beta")}
        sub["S0"] = x["S0"][i:i + 1][:, heads].cpu()
        sub["cu_seqlens"] = torch.tensor([0, b - a], dtype=torch.int32)
        ro, rS, _ = run_oracle(sub)
        report(f"split budget: sequence {i} ({b - a} tokens, heads {heads[:2]}..)",
               [("o", o[a:b][:, heads].cpu(), ro, (1,)), ("S_final", S[i:i + 1][:, heads].cpu(), rS)],
               TOL_BF16)


def test_bf16_without_initial_state_or_checkpoints():
    x = W.varlen_inputs(BASE, [300, 5, 129], H=8, seed=22)
    x["S0"] = None
    got = run_gpu(x)
    assert got[2] is None
    check("bf16 varlen no S0 no ckpt", x, got, run_oracle(x), TOL_BF16)


@pytest.mark.parametrize("dk,dv,chunk", [(16, 16, 16), (32, 64, 32), (64, 32, 64),
                                         (128, 128, 64), (16, 128, 16)])
def test_fp32_paths(dk, dv, chunk):
    import dataclasses
    base = dataclasses.replace(BASE, dk=dk, dv=dv)
    x = W.varlen_inputs(base, [70, 0, 128, 1, 200], H=3, seed=23, dtype=torch.float32)
    got = run_gpu(x, ckpt_every=64, chunk=chunk)
    check(f"fp32 varlen dk{dk} dv{dv} C{chunk}", x, got, run_oracle(x, 64), TOL_F32)


@pytest.mark.parametrize("B,H,T", [(1, 16, 700), (3, 64, 130)])
def test_uniform_lengths_equal_fixed_entry_point(B, H, T):
    # same kernels, same arithmetic: bit-identical to kda_prefill_fwd
    x = W.prefill_inputs(BASE, B=B, T=T, H=H)
    xd = to_dev(x)
    o_f, S_f = kda.kda_prefill_fwd(xd["q"], xd["k"], xd["v"], xd["log_alpha"], xd["beta"],
                                   xd["S0"])
    flat = lambda t: t.reshape(B * T, *t.shape[2:])
    cu = torch.arange(0, B * T + 1, T, dtype=torch.int32, device=DEV)
    o_v, S_v, _ = kda.kda_prefill_varlen(flat(xd["q"]), flat(xd["k"]), flat(xd["v"]),
                                         flat(xd["log_alpha"]), flat(xd["beta"]), cu, xd["S0"])
    torch.cuda.synchronize()
    assert torch.equal(flat(o_f), o_v)
    assert torch.equal(S_f, S_v)


def test_checkpoints_equal_prefix_final_states():
    # checkpoint j of a sequence is the final state of its first j*K tokens
    x = W.varlen_inputs(BASE, [640, 300], H=4, seed=24)
    o, S, Sc = run_gpu(x, ckpt_every=128)
    torch.cuda.synchronize()
    assert Sc.shape[0] == 640 // 128 + 300 // 128
    xd = to_dev(x)
    for j, n in enumerate([128, 256, 384, 512, 640]):
        sl = slice(0, n)
        _, Sp, _ = kda.kda_prefill_varlen(xd["q"][sl], xd["k"][sl], xd["v"][sl],
                                          xd["log_alpha"][sl], xd["beta"][sl],
                                          torch.tensor([0, n], dtype=torch.int32, device=DEV),
                                          xd["S0"][:1])
        torch.cuda.synchronize()
        assert torch.equal(Sp[0], Sc[j]), f"checkpoint {j}"


def test_out_of_order_offsets_are_clamped():
    # offsets outside [0, T] or decreasing: sequence i covers
    # [m_i, m_{i+1}), m_j = max(clamp(cu[0..j], 0, T)); rows outside every
    # sequence are not written
    x = W.varlen_inputs(BASE, [100, 100, 100], H=4, seed=25)
    T = 300
    bad = torch.tensor([10, 120, -60, 250, 999], dtype=torch.int32)   # N = 4
    x["cu_seqlens"] = bad
    x["S0"] = 0.02 * torch.randn((4, 4, 128, 128), generator=torch.Generator().manual_seed(3))
    m = np.maximum.accumulate(np.clip(bad.numpy(), 0, T))
    assert m.tolist() == [10, 120, 120, 250, 300]
    xd = to_dev(x)
    o = torch.full((T, 4, 128), 7.0, dtype=torch.bfloat16, device=DEV)
    o, S, _ = kda.kda_prefill_varlen(xd["q"], xd["k"], xd["v"], xd["log_alpha"], xd["beta"],
                                     xd["cu_seqlens"], xd["S0"], o=o)
    torch.cuda.synchronize()
    ro, rS, _ = run_oracle(x, cu=m.tolist())
    report("bf16 varlen clamped offsets", [("o", o[10:], ro[10:]), ("S_final", S, rS)],
           TOL_BF16)
    assert torch.all(o[:10] == 7.0)


def test_too_few_checkpoint_slots():
    x = W.varlen_inputs(BASE, [256, 192], H=2, seed=26)
    big = torch.full((8, 2, 128, 128), -3.0, device=DEV)
    view = big[:2]                              # 2 slots; 4 + 3 checkpoints exist
    o, S, Sc = run_gpu(x, ckpt_every=64, S_ckpt=view)
    ro, rS, rSc = run_oracle(x, 64)
    report("bf16 varlen 2 of 7 checkpoint slots", [("S_ckpt", Sc, rSc[:2]), ("S_final", S, rS)],
           TOL_BF16)
    assert torch.all(big[2:] == -3.0)           # nothing past the slots


def test_varlen_config_full_size_sampled():
    # the serving-style mix at full size in the benchmark's launch
    # configuration; the oracle checks the shortest sequences on every head
    c = W.VARLEN_CONFIGS["varlen"]
    lengths = W.varlen_lengths(c.total, c.len_lo, c.len_hi, c.seed)
    x = W.varlen_inputs(BASE, lengths, H=c.H, seed=c.seed)
    o, S, Sc = run_gpu(x, ckpt_every=c.ckpt_every)
    cu = x["cu_seqlens"].tolist()
    ck0 = np.concatenate([[0], np.cumsum([n // c.ckpt_every for n in lengths])])
    order = np.argsort(lengths)
    # the two shortest sequences on every head; the two longest (which the
    # split schedule cuts between the fused kernel and the state walk) on
    # two heads each, all tokens and checkpoints
    for i, heads in [(i, None) for i in order[:2]] + [(i, [3, 29]) for i in order[-2:]]:
        a, b = cu[i], cu[i + 1]
        hs = slice(None) if heads is None else heads
        sub = {n: x[n][a:b][:, hs] for n in ("q", "k", "v", "log_alpha", "beta")}
        sub["S0"] = x["S0"][i:i + 1][:, hs]
        sub["cu_seqlens"] = torch.tensor([0, b - a], dtype=torch.int32)
        ro, rS, rSc = run_oracle(sub, c.ckpt_every)
        pairs = [("o", o[a:b][:, hs].cpu(), ro, (1,)), ("S_final", S[i:i + 1][:, hs].cpu(), rS)]
        if rSc.shape[0]:
            pairs.append(("S_ckpt", Sc[ck0[i]:ck0[i + 1]][:, hs].cpu(), rSc))
        what = "all heads" if heads is None else f"heads {heads}"
        report(f"varlen full size: sequence {i} ({b - a} tokens, {what})", pairs, TOL_BF16)
    assert torch.isfinite(o.float()).all() and torch.isfinite(S).all()


def test_all_sequences_empty():
    x = W.varlen_inputs(BASE, [0, 0], H=2, seed=27)
    o, S, Sc = run_gpu(x, ckpt_every=64)
    assert o.shape == (0, 2, 128)
    assert torch.equal(S.cpu(), x["S0"])
