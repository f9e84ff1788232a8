"""Kimi Delta Attention hot path on MI355X: thin Python binding of libkda.so.

The functions below carry the C ABI's names (``include/kda.h``) and only
marshal arguments: they check devices, dtypes, shapes and contiguity, allocate
outputs with torch when the caller gives none, and pass raw device pointers
and the current HIP stream. Every step of the computation runs in the HIP
kernels behind the library; there is no other code path. If the library is
missing the calls raise.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

__all__ = [
    "KDAError", "lib_path", "load_library", "kda_status_string",
    "kda_prefill_workspace_size", "kda_prefill_fwd", "kda_prefill_varlen_workspace_size",
    "kda_prefill_varlen", "kda_decode_step", "kda_decode_multi", "kda_prefill_layer",
    "kda_decode_layer", "KDA_GATE_LOG", "KDA_GATE_BOUNDED", "KDA_GATE_SCALAR",
    "kda_prefill_fwd_noalloc", "KDA_NOALLOC_SCRATCH_BYTES",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libkda.so")
_lib = None

KDA_F32, KDA_BF16 = 0, 1
KDA_GATE_LOG, KDA_GATE_BOUNDED, KDA_GATE_SCALAR = 0, 1, 2


class _LayerOpts(ctypes.Structure):
    # kda_layer_opts in include/kda.h
    _fields_ = [("gate", ctypes.c_int), ("decay_bound", ctypes.c_float),
                ("l2norm_qk", ctypes.c_int), ("l2_eps", ctypes.c_float),
                ("out_gate", ctypes.c_void_p), ("out_weight", ctypes.c_void_p),
                ("out_eps", ctypes.c_float)]
_DTYPES = {torch.float32: KDA_F32, torch.bfloat16: KDA_BF16}


class KDAError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {kda_status_string(status)} (status {status})")
        self.status = status


def lib_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libkda.so (built by ``__graft_entry__.build()``); raise if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build the HIP library first "
                           "(python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, fp, i, sz = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.kda_status_string.argtypes = [i]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_prefill_workspace_size.argtypes = [i, i, i, i, i, i, i]
    lib.kda_prefill_workspace_size.restype = sz
    lib.kda_prefill_fwd.argtypes = [vp, vp, vp, fp, fp, fp, vp, fp, i, i, i, i, i, i, i,
                                    vp, sz, vp]
    lib.kda_prefill_fwd.restype = i
    lib.kda_prefill_varlen_workspace_size.argtypes = [i, i, i, i, i, i, i]
    lib.kda_prefill_varlen_workspace_size.restype = sz
    lib.kda_prefill_varlen.argtypes = [vp, vp, vp, fp, fp, fp, vp, fp, vp, i, i, i, i, i, i, i,
                                       fp, i, i, vp, sz, vp]
    lib.kda_prefill_varlen.restype = i
    lib.kda_prefill_layer.argtypes = [vp, vp, vp, vp, fp, fp, vp, fp, i, i, i, i, i, i, i,
                                      ctypes.POINTER(_LayerOpts), vp, sz, vp]
    lib.kda_prefill_layer.restype = i
    lib.kda_decode_layer.argtypes = [vp, vp, vp, vp, fp, fp, vp, i, i, i, i, i,
                                     ctypes.POINTER(_LayerOpts), vp]
    lib.kda_decode_layer.restype = i
    lib.kda_decode_step.argtypes = [vp, vp, vp, fp, fp, fp, vp, i, i, i, i, i, vp]
    lib.kda_decode_step.restype = i
    lib.kda_decode_multi.argtypes = [vp, vp, vp, fp, fp, fp, vp, vp, i, i, i, i, i, i, vp]
    lib.kda_decode_multi.restype = i
    lib.kda_prefill_fwd_noalloc.argtypes = [vp, vp, vp, fp, fp, fp, vp, fp, i, i, i, i, i, i, i,
                                            vp]
    lib.kda_prefill_fwd_noalloc.restype = i
    _lib = lib
    return lib


def kda_status_string(status: int) -> str:
    return load_library().kda_status_string(int(status)).decode()


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t: torch.Tensor, name: str, shape, dtype, device):
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(stream, device) -> ctypes.c_void_p:
    s = torch.cuda.current_stream(device) if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _empty(shape, dtype, device, stream) -> torch.Tensor:
    """A tensor this binding allocates for a call (an output the caller left
    out, or the workspace). torch's caching allocator ties it to the current
    stream; a call on another stream records that stream on it too, so that
    its memory is not handed out again, once the caller or this binding drops
    the tensor, before the call's kernels on that stream have finished."""
    t = torch.empty(shape, dtype=dtype, device=device)
    if stream is not None:
        t.record_stream(stream)
    return t


def kda_prefill_workspace_size(B: int, T: int, H: int, dk: int, dv: int,
                               dtype: torch.dtype, chunk: int = 64) -> int:
    return int(load_library().kda_prefill_workspace_size(B, T, H, dk, dv, _DTYPES[dtype], chunk))


def kda_prefill_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                    log_alpha: torch.Tensor, beta: torch.Tensor,
                    S0: Optional[torch.Tensor] = None, *, chunk: int = 64,
                    o: Optional[torch.Tensor] = None, S_final: Optional[torch.Tensor] = None,
                    want_state: bool = True, workspace: Optional[torch.Tensor] = None,
                    stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunked prefill. q,k,log_alpha [B,T,H,dk]; v [B,T,H,dv]; beta [B,T,H];
    S0 [B,H,dk,dv] fp32 or None. Returns (o [B,T,H,dv], S_final fp32 or None)."""
    lib = load_library()
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("kda_prefill_fwd needs GPU tensors")
    dt = q.dtype
    if dt not in _DTYPES:
        raise ValueError(f"unsupported dtype {dt}")
    _check(q, "q", (B, T, H, dk), dt, dev)
    _check(k, "k", (B, T, H, dk), dt, dev)
    _check(v, "v", (B, T, H, dv), dt, dev)
    _check(log_alpha, "log_alpha", (B, T, H, dk), torch.float32, dev)
    _check(beta, "beta", (B, T, H), torch.float32, dev)
    if S0 is not None:
        _check(S0, "S0", (B, H, dk, dv), torch.float32, dev)
    if o is None:
        o = _empty((B, T, H, dv), dt, dev, stream)
    _check(o, "o", (B, T, H, dv), dt, dev)
    if S_final is None and want_state:
        S_final = _empty((B, H, dk, dv), torch.float32, dev, stream)
    if S_final is not None:
        _check(S_final, "S_final", (B, H, dk, dv), torch.float32, dev)
    ws_bytes = kda_prefill_workspace_size(B, T, H, dk, dv, dt, chunk)
    if ws_bytes and (workspace is None or workspace.numel() * workspace.element_size() < ws_bytes):
        workspace = _empty(ws_bytes, torch.uint8, dev, stream)
    wsz = 0 if workspace is None else workspace.numel() * workspace.element_size()
    with torch.cuda.device(dev):
        st = lib.kda_prefill_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S0),
                                 _ptr(o), _ptr(S_final), B, T, H, dk, dv, _DTYPES[dt], chunk,
                                 _ptr(workspace), wsz, _stream(stream, dev))
    if st != 0:
        raise KDAError(st, "kda_prefill_fwd")
    return o, S_final


KDA_NOALLOC_SCRATCH_BYTES = 80 << 20   # include/kda.h


def kda_prefill_fwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                            log_alpha: torch.Tensor, beta: torch.Tensor,
                            S0: Optional[torch.Tensor], o: torch.Tensor,
                            S_final: Optional[torch.Tensor], *, chunk: int = 64,
                            stream=None) -> None:
    """kda_prefill_fwd through the entry point that allocates nothing: the
    caller passes the outputs, and the library's static device scratch serves
    as the workspace. Layouts as kda_prefill_fwd."""
    lib = load_library()
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("kda_prefill_fwd_noalloc needs GPU tensors")
    dt = q.dtype
    if dt not in _DTYPES:
        raise ValueError(f"unsupported dtype {dt}")
    _check(q, "q", (B, T, H, dk), dt, dev)
    _check(k, "k", (B, T, H, dk), dt, dev)
    _check(v, "v", (B, T, H, dv), dt, dev)
    _check(log_alpha, "log_alpha", (B, T, H, dk), torch.float32, dev)
    _check(beta, "beta", (B, T, H), torch.float32, dev)
    if S0 is not None:
        _check(S0, "S0", (B, H, dk, dv), torch.float32, dev)
    _check(o, "o", (B, T, H, dv), dt, dev)
    if S_final is not None:
        _check(S_final, "S_final", (B, H, dk, dv), torch.float32, dev)
    with torch.cuda.device(dev):
        st = lib.kda_prefill_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                                         _ptr(S0), _ptr(o), _ptr(S_final), B, T, H, dk, dv,
                                         _DTYPES[dt], chunk, _stream(stream, dev))
    if st != 0:
        raise KDAError(st, "kda_prefill_fwd_noalloc")


def kda_prefill_varlen_workspace_size(N: int, T_total: int, H: int, dk: int, dv: int,
                                      dtype: torch.dtype, chunk: int = 64) -> int:
    return int(load_library().kda_prefill_varlen_workspace_size(N, T_total, H, dk, dv,
                                                                _DTYPES[dtype], chunk))


def kda_prefill_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                       log_alpha: torch.Tensor, beta: torch.Tensor, cu_seqlens: torch.Tensor,
                       S0: Optional[torch.Tensor] = None, *, ckpt_every: int = 0,
                       ckpt_slots: Optional[int] = None, chunk: int = 64,
                       o: Optional[torch.Tensor] = None, S_final: Optional[torch.Tensor] = None,
                       S_ckpt: Optional[torch.Tensor] = None, want_state: bool = True,
                       workspace: Optional[torch.Tensor] = None, stream=None
                       ) -> Tuple[torch.Tensor, Optional[torch.Tensor], Optional[torch.Tensor]]:
    """Packed variable-length prefill. q,k,log_alpha [T,H,dk]; v [T,H,dv]; beta [T,H];
    cu_seqlens int32 [N+1] on the device; S0 [N,H,dk,dv] fp32 or None. With
    ckpt_every > 0 (a multiple of 64) the state after every ckpt_every tokens
    of each sequence goes to S_ckpt [ckpt_slots,H,dk,dv] (default
    T // ckpt_every slots, allocated uninitialised: only the first
    sum(len_i // ckpt_every) of them are written). Returns (o [T,H,dv],
    S_final or None, S_ckpt or None)."""
    lib = load_library()
    T, H, dk = q.shape
    dv = v.shape[-1]
    N = cu_seqlens.shape[0] - 1
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("kda_prefill_varlen needs GPU tensors")
    if N < 0:
        raise ValueError("cu_seqlens needs N + 1 >= 1 entries")
    dt = q.dtype
    if dt not in _DTYPES:
        raise ValueError(f"unsupported dtype {dt}")
    _check(q, "q", (T, H, dk), dt, dev)
    _check(k, "k", (T, H, dk), dt, dev)
    _check(v, "v", (T, H, dv), dt, dev)
    _check(log_alpha, "log_alpha", (T, H, dk), torch.float32, dev)
    _check(beta, "beta", (T, H), torch.float32, dev)
    _check(cu_seqlens, "cu_seqlens", (N + 1,), torch.int32, dev)
    if S0 is not None:
        _check(S0, "S0", (N, H, dk, dv), torch.float32, dev)
    if o is None:
        o = _empty((T, H, dv), dt, dev, stream)
    _check(o, "o", (T, H, dv), dt, dev)
    if S_final is None and want_state:
        S_final = _empty((N, H, dk, dv), torch.float32, dev, stream)
    if S_final is not None:
        _check(S_final, "S_final", (N, H, dk, dv), torch.float32, dev)
    if ckpt_every > 0:
        if ckpt_slots is None:
            ckpt_slots = S_ckpt.shape[0] if S_ckpt is not None else max(T // ckpt_every, 1)
        if S_ckpt is None:
            S_ckpt = _empty((ckpt_slots, H, dk, dv), torch.float32, dev, stream)
        _check(S_ckpt, "S_ckpt", (ckpt_slots, H, dk, dv), torch.float32, dev)
    else:
        ckpt_slots, S_ckpt = 0, None
    ws_bytes = kda_prefill_varlen_workspace_size(N, T, H, dk, dv, dt, chunk)
    if ws_bytes and (workspace is None or workspace.numel() * workspace.element_size() < ws_bytes):
        workspace = _empty(ws_bytes, torch.uint8, dev, stream)
    wsz = 0 if workspace is None else workspace.numel() * workspace.element_size()
    with torch.cuda.device(dev):
        st = lib.kda_prefill_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                                    _ptr(S0), _ptr(o), _ptr(S_final), _ptr(cu_seqlens), N, T, H,
                                    dk, dv, _DTYPES[dt], chunk, _ptr(S_ckpt), int(ckpt_every),
                                    int(ckpt_slots), _ptr(workspace), wsz, _stream(stream, dev))
    if st != 0:
        raise KDAError(st, "kda_prefill_varlen")
    return o, S_final, S_ckpt


def kda_decode_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                    log_alpha: torch.Tensor, beta: torch.Tensor, S: torch.Tensor, *,
                    o: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """One decode step; S [B,H,dk,dv] fp32 is updated in place. Returns o [B,H,dv]."""
    lib = load_library()
    B, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("kda_decode_step needs GPU tensors")
    dt = q.dtype
    if dt not in _DTYPES:
        raise ValueError(f"unsupported dtype {dt}")
    _check(q, "q", (B, H, dk), dt, dev)
    _check(k, "k", (B, H, dk), dt, dev)
    _check(v, "v", (B, H, dv), dt, dev)
    _check(log_alpha, "log_alpha", (B, H, dk), torch.float32, dev)
    _check(beta, "beta", (B, H), torch.float32, dev)
    _check(S, "S", (B, H, dk, dv), torch.float32, dev)
    if o is None:
        o = _empty((B, H, dv), dt, dev, stream)
    _check(o, "o", (B, H, dv), dt, dev)
    with torch.cuda.device(dev):
        st = lib.kda_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S),
                                 _ptr(o), B, H, dk, dv, _DTYPES[dt], _stream(stream, dev))
    if st != 0:
        raise KDAError(st, "kda_decode_step")
    return o


def kda_decode_multi(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                     log_alpha: torch.Tensor, beta: torch.Tensor, S: torch.Tensor, *,
                     n_commit: Optional[torch.Tensor] = None,
                     o: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """T tokens per sequence from the live state S [B,H,dk,dv] (fp32): returns
    o [B,T,H,dv] for every token and overwrites S[b] with the state after the
    first n_commit[b] tokens (int32 [B] on the device; None = all T; 0 leaves
    S[b] untouched)."""
    lib = load_library()
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("kda_decode_multi needs GPU tensors")
    dt = q.dtype
    if dt not in _DTYPES:
        raise ValueError(f"unsupported dtype {dt}")
    _check(q, "q", (B, T, H, dk), dt, dev)
    _check(k, "k", (B, T, H, dk), dt, dev)
    _check(v, "v", (B, T, H, dv), dt, dev)
    _check(log_alpha, "log_alpha", (B, T, H, dk), torch.float32, dev)
    _check(beta, "beta", (B, T, H), torch.float32, dev)
    _check(S, "S", (B, H, dk, dv), torch.float32, dev)
    if n_commit is not None:
        _check(n_commit, "n_commit", (B,), torch.int32, dev)
    if o is None:
        o = _empty((B, T, H, dv), dt, dev, stream)
    _check(o, "o", (B, T, H, dv), dt, dev)
    with torch.cuda.device(dev):
        st = lib.kda_decode_multi(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S),
                                  _ptr(o), _ptr(n_commit), B, T, H, dk, dv, _DTYPES[dt],
                                  _stream(stream, dev))
    if st != 0:
        raise KDAError(st, "kda_decode_multi")
    return o


def _layer_opts(gate_mode, decay_bound, l2norm, l2_eps, z, w, out_eps):
    return _LayerOpts(int(gate_mode), float(decay_bound), int(bool(l2norm)), float(l2_eps),
                      None if z is None else z.data_ptr(), None if w is None else w.data_ptr(),
                      float(out_eps))


def _check_layer_extra(gate, gate_mode, tok_shape, dk, dv, dt, dev, z, w):
    if gate_mode == KDA_GATE_LOG:
        _check(gate, "gate", tok_shape + (dk,), torch.float32, dev)
    elif gate_mode == KDA_GATE_BOUNDED:
        _check(gate, "gate", tok_shape + (dk,), dt, dev)
    elif gate_mode == KDA_GATE_SCALAR:
        _check(gate, "gate", tok_shape, torch.float32, dev)
    else:
        raise ValueError(f"unknown gate mode {gate_mode}")
    if z is not None:
        _check(z, "z", tok_shape + (dv,), dt, dev)
    if w is not None:
        _check(w, "w", (dv,), torch.float32, dev)


def kda_prefill_layer(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, gate: torch.Tensor,
                      beta: torch.Tensor, S0: Optional[torch.Tensor] = None, *,
                      gate_mode: int = KDA_GATE_LOG, decay_bound: float = 5.0,
                      l2norm: bool = False, l2_eps: float = 1e-6,
                      z: Optional[torch.Tensor] = None, w: Optional[torch.Tensor] = None,
                      out_eps: float = 1e-6, chunk: int = 64,
                      o: Optional[torch.Tensor] = None, S_final: Optional[torch.Tensor] = None,
                      want_state: bool = True, workspace: Optional[torch.Tensor] = None,
                      stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Prefill in the layer form: q, k raw or normalised ([B,T,H,dk]), gate
    per gate_mode (fp32 log-decay [B,T,H,dk]; pre-activation g in the q dtype
    [B,T,H,dk]; fp32 per-head log-decay [B,T,H]), optional epilogue with z
    [B,T,H,dv] and w [dv]. Returns (o, S_final or None)."""
    lib = load_library()
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("kda_prefill_layer needs GPU tensors")
    dt = q.dtype
    if dt not in _DTYPES:
        raise ValueError(f"unsupported dtype {dt}")
    _check(q, "q", (B, T, H, dk), dt, dev)
    _check(k, "k", (B, T, H, dk), dt, dev)
    _check(v, "v", (B, T, H, dv), dt, dev)
    _check(beta, "beta", (B, T, H), torch.float32, dev)
    _check_layer_extra(gate, gate_mode, (B, T, H), dk, dv, dt, dev, z, w)
    if S0 is not None:
        _check(S0, "S0", (B, H, dk, dv), torch.float32, dev)
    if o is None:
        o = _empty((B, T, H, dv), dt, dev, stream)
    _check(o, "o", (B, T, H, dv), dt, dev)
    if S_final is None and want_state:
        S_final = _empty((B, H, dk, dv), torch.float32, dev, stream)
    if S_final is not None:
        _check(S_final, "S_final", (B, H, dk, dv), torch.float32, dev)
    ws_bytes = kda_prefill_workspace_size(B, T, H, dk, dv, dt, chunk)
    if ws_bytes and (workspace is None or workspace.numel() * workspace.element_size() < ws_bytes):
        workspace = _empty(ws_bytes, torch.uint8, dev, stream)
    wsz = 0 if workspace is None else workspace.numel() * workspace.element_size()
    opts = _layer_opts(gate_mode, decay_bound, l2norm, l2_eps, z, w, out_eps)
    with torch.cuda.device(dev):
        st = lib.kda_prefill_layer(_ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(beta), _ptr(S0),
                                   _ptr(o), _ptr(S_final), B, T, H, dk, dv, _DTYPES[dt], chunk,
                                   ctypes.byref(opts), _ptr(workspace), wsz, _stream(stream, dev))
    if st != 0:
        raise KDAError(st, "kda_prefill_layer")
    return o, S_final


def kda_decode_layer(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, gate: torch.Tensor,
                     beta: torch.Tensor, S: torch.Tensor, *, gate_mode: int = KDA_GATE_LOG,
                     decay_bound: float = 5.0, l2norm: bool = False, l2_eps: float = 1e-6,
                     z: Optional[torch.Tensor] = None, w: Optional[torch.Tensor] = None,
                     out_eps: float = 1e-6, o: Optional[torch.Tensor] = None,
                     stream=None) -> torch.Tensor:
    """One decode step in the layer form (shapes as kda_decode_step, gate per
    gate_mode: [B,H,dk] or [B,H]); S updated in place. Returns o [B,H,dv]."""
    lib = load_library()
    B, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("kda_decode_layer needs GPU tensors")
    dt = q.dtype
    if dt not in _DTYPES:
        raise ValueError(f"unsupported dtype {dt}")
    _check(q, "q", (B, H, dk), dt, dev)
    _check(k, "k", (B, H, dk), dt, dev)
    _check(v, "v", (B, H, dv), dt, dev)
    _check(beta, "beta", (B, H), torch.float32, dev)
    _check(S, "S", (B, H, dk, dv), torch.float32, dev)
    _check_layer_extra(gate, gate_mode, (B, H), dk, dv, dt, dev, z, w)
    if o is None:
        o = _empty((B, H, dv), dt, dev, stream)
    _check(o, "o", (B, H, dv), dt, dev)
    opts = _layer_opts(gate_mode, decay_bound, l2norm, l2_eps, z, w, out_eps)
    with torch.cuda.device(dev):
        st = lib.kda_decode_layer(_ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(beta), _ptr(S),
                                  _ptr(o), B, H, dk, dv, _DTYPES[dt], ctypes.byref(opts),
                                  _stream(stream, dev))
    if st != 0:
        raise KDAError(st, "kda_decode_layer")
    return o
