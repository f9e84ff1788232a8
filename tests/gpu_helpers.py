"""Shared helpers of the GPU parity tests (no test cases here)."""
import numpy as np
import torch

import oracle

TOL_F32 = 1e-5   # fp32 inputs, fp32 arithmetic
TOL_BF16 = 2e-2  # bf16 inputs, fp32 accumulation and state

DEV = torch.device("cuda:0")


def to_dev(x: dict) -> dict:
    return {n: (t.to(DEV) if t is not None else None) for n, t in x.items()}


def to_host(x: dict) -> dict:
    return {n: (t.detach().cpu() if t is not None else None) for n, t in x.items()}


def report(label: str, pairs, tol: float):
    """pairs: [(name, gpu_tensor, oracle_array)]; asserts max rel-L2 <= tol."""
    errs = {}
    for name, got, ref in pairs:
        errs[name] = oracle.rel_l2(got.detach().cpu() if hasattr(got, "detach") else got, ref)
    msg = " ".join(f"{n}={e:.3e}" for n, e in errs.items())
    print(f"[parity] {label}: {msg} (tol {tol:g})", flush=True)
    for n, e in errs.items():
        assert np.isfinite(e) and e <= tol, f"{label}: {n} rel-L2 {e:.3e} > {tol:g}"
    return errs
