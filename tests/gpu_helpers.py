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


def _f64(x):
    if hasattr(x, "detach"):
        x = x.detach().cpu()
        return x.double().numpy()
    return np.asarray(x, dtype=np.float64)


def head_axes(name: str, ndim: int):
    """Axes that index one (sequence, head) recurrence in a 4-D tensor of this
    name: outputs [B, T, H, d] -> (0, 2); states [B, H, dk, dv] -> (0, 1).
    None otherwise (a caller can name the axes of other layouts)."""
    if name.startswith("S") and ndim == 4:
        return (0, 1)
    if name.startswith("o") and ndim == 4:
        return (0, 2)
    return None


def per_head_rel_l2(got, ref, axes):
    """Largest rel-L2 over the (sequence, head) slices (the recurrences are
    independent per head, so a head is the natural unit of error)."""
    x, r = _f64(got), _f64(ref)
    if x.size == 0:          # no tokens (or no heads): nothing to compare
        return 0.0, 0
    rest = [a for a in range(x.ndim) if a not in axes]
    x = np.transpose(x, list(axes) + rest).reshape(-1, int(np.prod([x.shape[a] for a in rest])))
    r = np.transpose(r, list(axes) + rest).reshape(x.shape)
    nr = np.linalg.norm(r, axis=1)
    nd = np.linalg.norm(x - r, axis=1)
    amax = np.max(np.abs(x - r), axis=1)
    e = np.where(nr > 0, nd / np.where(nr > 0, nr, 1.0), amax)
    i = int(np.argmax(e))
    return float(e[i]), i


def report(label: str, pairs, tol: float):
    """pairs: [(name, gpu_tensor, oracle_array[, head_axes])]. Asserts, for
    each pair, the rel-L2 over the whole tensor and the largest rel-L2 over
    its (sequence, head) slices, both <= tol. The head axes default to
    head_axes(name, ndim)."""
    errs, worst = {}, {}
    for pair in pairs:
        name, got, ref = pair[:3]
        g = got.detach().cpu() if hasattr(got, "detach") else got
        errs[name] = oracle.rel_l2(g, ref)
        axes = pair[3] if len(pair) > 3 else head_axes(name, np.ndim(ref))
        if axes is not None:
            worst[name] = per_head_rel_l2(g, ref, axes)
    msg = " ".join(f"{n}={e:.3e}" for n, e in errs.items())
    if worst:
        msg += " | worst head " + " ".join(f"{n}={e:.3e}@{i}" for n, (e, i) in worst.items())
    print(f"[parity] {label}: {msg} (tol {tol:g})", flush=True)
    for n, e in errs.items():
        assert np.isfinite(e) and e <= tol, f"{label}: {n} rel-L2 {e:.3e} > {tol:g}"
    for n, (e, i) in worst.items():
        assert np.isfinite(e) and e <= tol, f"{label}: {n} head slice {i} rel-L2 {e:.3e} > {tol:g}"
    return errs
