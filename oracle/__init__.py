"""KDA fp64 oracle — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The GPU product path never imports it,
and this package imports nothing from the product package.

``prefill_f64`` / ``decode_f64`` wrap the plain C token-by-token recurrence in
``kda_oracle.c`` (definition: Kimi K3 blog, section "Kimi Delta Attention").
``prefill_varlen_f64`` runs the same recurrence over packed sequences and
records the state at fixed token intervals (the checkpoints a prefix cache
keeps: "Kimi K3: the manos...", section "KDA Prefix Cache Management").
``chunk_form`` holds an independent fp64 NumPy statement of the chunked
unrolling (FlashKDA algorithm, "Kimi K3: the manos..." section "FlashKDA
Algorithm"), used by tests only to pin the chunk algebra against the step form.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libkda_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (-O2, no fast-math, libm exp)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
               os.path.join(_HERE, "kda_oracle.c"), "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        dp = ctypes.POINTER(ctypes.c_double)
        L = ctypes.c_long
        lib.kda_oracle_prefill_f64.argtypes = [dp] * 8 + [L] * 5 + [ctypes.c_int]
        lib.kda_oracle_prefill_f64.restype = ctypes.c_int
        lib.kda_oracle_decode_f64.argtypes = [dp] * 7 + [L] * 4 + [ctypes.c_int]
        lib.kda_oracle_decode_f64.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f64(x):
    """Exact widening of a torch tensor (bf16/fp32/fp64) or array to contiguous fp64."""
    if x is None:
        return None
    if hasattr(x, "detach"):
        import torch
        x = x.detach().to("cpu", torch.float64).contiguous().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _threads(n):
    if n is None:
        n = os.cpu_count() or 1
    return int(max(1, min(n, 64)))


def prefill_f64(q, k, v, log_alpha, beta, S0=None, nthreads=None, want_o=True):
    """Token-by-token fp64 recurrence over [B,T,H,*] inputs.
    Returns (o [B,T,H,dv] or None, S_final [B,H,dk,dv])."""
    q, k, v, la, beta, S0 = map(_f64, (q, k, v, log_alpha, beta, S0))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == q.shape and la.shape == q.shape
    assert v.shape == (B, T, H, dv) and beta.shape == (B, T, H)
    if S0 is not None:
        assert S0.shape == (B, H, dk, dv)
    o = np.zeros((B, T, H, dv), np.float64) if want_o else None
    S = np.zeros((B, H, dk, dv), np.float64)
    rc = _load().kda_oracle_prefill_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(la), _ptr(beta),
                                        _ptr(S0), _ptr(o), _ptr(S), B, T, H, dk, dv,
                                        _threads(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return o, S


def prefill_varlen_f64(q, k, v, log_alpha, beta, cu_seqlens, S0=None, ckpt_every=0,
                       nthreads=None):
    """Packed sequences: q, k, log_alpha [T,H,dk]; v [T,H,dv]; beta [T,H];
    sequence i is tokens cu_seqlens[i] .. cu_seqlens[i+1] - 1 (offsets must be
    non-decreasing inside [0, T]) and starts from S0[i] (zeros if S0 is None).
    With ckpt_every > 0 the state after every ckpt_every tokens of each
    sequence is recorded, sequence by sequence in order.
    Returns (o [T,H,dv], S_final [N,H,dk,dv], S_ckpt [n_ckpt,H,dk,dv])."""
    q, k, v, la, beta, S0 = map(_f64, (q, k, v, log_alpha, beta, S0))
    cu = [int(x) for x in (cu_seqlens.tolist() if hasattr(cu_seqlens, "tolist") else cu_seqlens)]
    T, H, dk = q.shape
    dv = v.shape[-1]
    N = len(cu) - 1
    if cu[0] < 0 or cu[-1] > T or any(b < a for a, b in zip(cu, cu[1:])):
        raise ValueError("cu_seqlens must be non-decreasing inside [0, T]")
    o = np.zeros((T, H, dv), np.float64)
    S_final = np.zeros((N, H, dk, dv), np.float64)
    ckpts = []
    for i in range(N):
        S = np.zeros((1, H, dk, dv)) if S0 is None else S0[i:i + 1].copy()
        a, b = cu[i], cu[i + 1]
        # cut at every checkpoint; the token loop carries S exactly across cuts
        cuts = list(range(a, b, ckpt_every)) + [b] if ckpt_every > 0 else [a, b]
        for s0, s1 in zip(cuts, cuts[1:]):
            if s1 == s0:
                continue
            seg = slice(s0, s1)
            oi, S = prefill_f64(q[None, seg], k[None, seg], v[None, seg], la[None, seg],
                                beta[None, seg], S, nthreads=nthreads)
            o[seg] = oi[0]
            if ckpt_every > 0 and (s1 - a) % ckpt_every == 0:
                ckpts.append(S[0].copy())
        S_final[i] = S[0]
    S_ckpt = np.stack(ckpts) if ckpts else np.zeros((0, H, dk, dv), np.float64)
    return o, S_final, S_ckpt


def decode_f64(q, k, v, log_alpha, beta, S, nthreads=None):
    """One decode step on a copy of S [B,H,dk,dv]. Returns (o [B,H,dv], S_new)."""
    q, k, v, la, beta = map(_f64, (q, k, v, log_alpha, beta))
    S = _f64(S).copy()
    B, H, dk = q.shape
    dv = v.shape[-1]
    assert S.shape == (B, H, dk, dv)
    o = np.zeros((B, H, dv), np.float64)
    rc = _load().kda_oracle_decode_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(la), _ptr(beta),
                                       _ptr(S), _ptr(o), B, H, dk, dv, _threads(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return o, S


def rel_l2(x, ref) -> float:
    """||x - ref||_2 / ||ref||_2 over the whole tensor, in fp64 (absolute
    max error where the reference is all zeros)."""
    x = _f64(x)
    ref = _f64(ref)
    nr = float(np.linalg.norm(ref.ravel()))
    diff = float(np.linalg.norm((x - ref).ravel()))
    if nr == 0.0:
        return float(np.max(np.abs(x - ref))) if x.size else 0.0
    return diff / nr
