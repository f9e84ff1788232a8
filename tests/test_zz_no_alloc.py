"""kda_prefill_fwd_noalloc (the entry point that allocates nothing, for
callers that cannot call hipMalloc) against kda_prefill_fwd with a caller
workspace, through the C ABI: two calls in a row on the same GPU, the second
on a smaller input, each compared element by element (same kernels, same
inputs: the results must be identical), and calls whose usual workspace
exceeds the static array, which run in shorter pieces."""
import pytest
import torch

import gated_delta_rule_22_amd as kda
import oracle
import workloads as W
from gpu_helpers import DEV, TOL_BF16, report, to_dev

pytestmark = pytest.mark.gpu


def _both(x):
    xd = to_dev(x)
    o_ref, S_ref = kda.kda_prefill_fwd(xd["q"], xd["k"], xd["v"], xd["log_alpha"], xd["beta"],
                                       xd["S0"])
    o = torch.full_like(o_ref, float("nan"))
    S = torch.full_like(S_ref, float("nan"))
    kda.kda_prefill_fwd_noalloc(xd["q"], xd["k"], xd["v"], xd["log_alpha"], xd["beta"],
                                xd["S0"], o, S)
    torch.cuda.synchronize()
    return o, S, o_ref, S_ref


def test_noalloc_matches_workspace_entry_point_twice():
    c = W.PREFILL_CONFIGS["prefill"]
    # first call: the full 4K configuration (73.9 MB of scratch records)
    x = W.prefill_inputs(c)
    assert kda.kda_prefill_workspace_size(1, c.T, c.H, 128, 128, torch.bfloat16) > (64 << 20)
    o, S, o_ref, S_ref = _both(x)
    assert torch.equal(o, o_ref) and torch.equal(S, S_ref)
    ro, rS = oracle.prefill_f64(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], None)
    report("noalloc B1 H16 T4096", [("o", o, ro), ("S", S, rS)], TOL_BF16)
    # second call, smaller and ragged, with a carried state: the scratch keeps
    # the first call's records, which must not leak into this one
    cb = W.PREFILL_CONFIGS["batched"]
    x = W.prefill_inputs(cb, B=1, T=333, H=5, seed=77)
    o, S, o_ref, S_ref = _both(x)
    assert torch.equal(o, o_ref) and torch.equal(S, S_ref)
    ro, rS = oracle.prefill_f64(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["S0"])
    report("noalloc B1 H5 T333 after a larger call", [("o", o, ro), ("S", S, rS)], TOL_BF16)


def test_noalloc_paths_without_scratch():
    # many heads (fused kernel) and fp32 (generic kernel) need no workspace
    cb = W.PREFILL_CONFIGS["batched"]
    x = W.prefill_inputs(cb, B=2, T=130, H=64, seed=78)
    o, S, o_ref, S_ref = _both(x)
    assert torch.equal(o, o_ref) and torch.equal(S, S_ref)
    x = W.prefill_inputs(cb, B=1, T=70, H=3, seed=79, dtype=torch.float32)
    o, S, o_ref, S_ref = _both(x)
    assert torch.equal(o, o_ref) and torch.equal(S, S_ref)


@pytest.mark.parametrize("T,H", [(8192, 16), (65536, 4)])
def test_noalloc_long_calls_run_in_shorter_pieces(T, H):
    # calls whose usual workspace exceeds the 80 MiB array (147.8 MB and
    # 222 MB) run the split path in pieces short enough for one to fit (71
    # chunks, 289 chunks): the same kernels on the same chunks, so the
    # results equal kda_prefill_fwd's bit for bit
    c = W.PREFILL_CONFIGS["prefill"]
    assert kda.kda_prefill_workspace_size(1, T, H, 128, 128, torch.bfloat16) > \
        kda.KDA_NOALLOC_SCRATCH_BYTES
    x = W.prefill_inputs(c, T=T, H=H, seed=80)
    o, S, o_ref, S_ref = _both(x)
    assert torch.equal(o, o_ref) and torch.equal(S, S_ref)
