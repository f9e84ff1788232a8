"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before any launch."""
import ctypes
import os
import re

import pytest

import gated_delta_rule_22_amd as kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")

OK, INVALID, UNSUPPORTED, WORKSPACE, HIPERR, SCRATCH = 0, 1, 2, 3, 4, 5


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kda.lib_path()):
        import __graft_entry__
        __graft_entry__.build()
    return kda.load_library()


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    syms = declared_symbols()
    assert set(syms) == {"kda_prefill_workspace_size", "kda_prefill_fwd",
                         "kda_prefill_varlen_workspace_size", "kda_prefill_varlen",
                         "kda_prefill_layer", "kda_decode_layer",
                         "kda_decode_step", "kda_decode_multi", "kda_status_string",
                         "kda_prefill_fwd_noalloc"}
    for s in syms:
        assert hasattr(lib, s), s


def test_status_strings(lib):
    for code in (OK, INVALID, UNSUPPORTED, WORKSPACE, HIPERR, SCRATCH, 99):
        assert kda.kda_status_string(code)
    assert kda.kda_status_string(OK) == "ok"


# Fake, 256-byte-spaced device addresses: validation must reject before any use.
# The calls below pass them to the real entry points, so they run only where
# no GPU is visible: if host validation ever regressed there, a launch would
# fail with KDA_ERR_HIP instead of touching the made-up addresses on a card.
BASE = 1 << 40
no_gpu = pytest.mark.skipif(os.path.exists("/dev/kfd"),
                            reason="fake device addresses: run only where no GPU is visible")


def P(i, off=0):
    return ctypes.c_void_p(BASE + (i << 30) + off)


def prefill(lib, *, q=P(0), k=P(1), v=P(2), la=P(3), beta=P(4), S0=P(5), o=P(6), Sf=P(7),
            B=1, T=64, H=2, dk=128, dv=128, dt=1, chunk=64, ws=P(10), ws_bytes=1 << 30):
    return lib.kda_prefill_fwd(q, k, v, la, beta, S0, o, Sf, B, T, H, dk, dv, dt, chunk,
                               ws, ws_bytes, None)


def decode(lib, *, q=P(0), k=P(1), v=P(2), la=P(3), beta=P(4), S=P(5), o=P(6),
           B=2, H=2, dk=128, dv=128, dt=1):
    return lib.kda_decode_step(q, k, v, la, beta, S, o, B, H, dk, dv, dt, None)


@no_gpu
def test_prefill_rejects(lib):
    assert prefill(lib, B=-1) == INVALID
    assert prefill(lib, T=-5) == INVALID
    assert prefill(lib, H=-1) == INVALID
    assert prefill(lib, dk=48) == UNSUPPORTED
    assert prefill(lib, dv=256) == UNSUPPORTED
    assert prefill(lib, chunk=128) == UNSUPPORTED
    assert prefill(lib, chunk=8) == UNSUPPORTED
    assert prefill(lib, dt=7) == UNSUPPORTED
    for name in ("q", "k", "v", "la", "beta", "o"):
        assert prefill(lib, **{name: None}) == INVALID, name
    for name in ("q", "k", "v", "la", "beta", "S0", "o", "Sf"):
        assert prefill(lib, **{name: P(8, 4)}) == INVALID, name   # misaligned
    # o overlapping an input, S_final overlapping an input other than S0
    assert prefill(lib, o=P(0, 256)) == INVALID
    assert prefill(lib, Sf=P(2, 1024)) == INVALID
    assert prefill(lib, Sf=P(5, 256)) == INVALID     # partial overlap with S0
    assert prefill(lib, o=P(7)) == INVALID           # o overlapping S_final


@no_gpu
def test_prefill_empty_batch_is_noop(lib):
    # nothing to do: returns before touching the device
    assert prefill(lib, B=0) == OK
    assert prefill(lib, H=0, q=None, k=None) == OK


def test_workspace_query(lib):
    # many heads: fused kernel, no workspace; few heads: chunk-parallel prep
    assert lib.kda_prefill_workspace_size(8, 8192, 32, 128, 128, 1, 64) == 0
    n = lib.kda_prefill_workspace_size(1, 4096, 16, 128, 128, 1, 64)
    assert n > 0 and n % 256 == 0
    assert lib.kda_prefill_workspace_size(1, 4096 + 1, 16, 128, 128, 1, 64) > n  # ragged tail
    assert lib.kda_prefill_workspace_size(1, 4096, 16, 128, 128, 0, 64) == 0    # fp32 path
    assert lib.kda_prefill_workspace_size(1, 0, 16, 128, 128, 1, 64) == 0


@no_gpu
def test_workspace_rejects(lib):
    need = lib.kda_prefill_workspace_size(1, 64, 2, 128, 128, 1, 64)
    assert prefill(lib, ws=None, ws_bytes=0) == WORKSPACE
    assert prefill(lib, ws=P(10), ws_bytes=need - 1) == WORKSPACE
    assert prefill(lib, ws=P(10, 8), ws_bytes=need) == INVALID     # misaligned
    assert prefill(lib, ws=P(0, 512), ws_bytes=need) == INVALID    # overlaps q
    assert prefill(lib, ws=P(6), ws_bytes=need) == INVALID         # overlaps o


@no_gpu
def test_decode_rejects(lib):
    assert decode(lib, B=-1) == INVALID
    assert decode(lib, dk=24) == UNSUPPORTED
    assert decode(lib, dt=3) == UNSUPPORTED
    for name in ("q", "k", "v", "la", "beta", "S", "o"):
        assert decode(lib, **{name: None}) == INVALID, name
        assert decode(lib, **{name: P(9, 8)}) == INVALID, name
    assert decode(lib, o=P(5, 512)) == INVALID       # o inside S
    assert decode(lib, S=P(1, 64)) == INVALID        # S overlapping k
    assert decode(lib, B=0) == OK


def multi(lib, *, q=P(0), k=P(1), v=P(2), la=P(3), beta=P(4), S=P(5), o=P(6), n=P(7),
          B=2, T=4, H=2, dk=128, dv=128, dt=1):
    return lib.kda_decode_multi(q, k, v, la, beta, S, o, n, B, T, H, dk, dv, dt, None)


@no_gpu
def test_decode_multi_rejects(lib):
    assert multi(lib, T=-1) == INVALID
    assert multi(lib, dv=48) == UNSUPPORTED
    assert multi(lib, dt=2) == UNSUPPORTED
    for name in ("q", "k", "v", "la", "beta", "S", "o"):
        assert multi(lib, **{name: None}) == INVALID, name
        assert multi(lib, **{name: P(9, 8)}) == INVALID, name
    assert multi(lib, n=P(7, 2)) == INVALID          # n_commit not 4-byte aligned
    assert multi(lib, o=P(7, 0)) == INVALID          # o overlapping n_commit
    assert multi(lib, S=P(0, 256)) == INVALID        # S overlapping q
    assert multi(lib, o=P(5, 64)) == INVALID         # o inside S
    assert multi(lib, T=0) == OK                     # nothing to do
    assert multi(lib, B=0) == OK


def varlen(lib, *, q=P(0), k=P(1), v=P(2), la=P(3), beta=P(4), S0=P(5), o=P(6), Sf=P(7),
           cu=P(8), N=3, T=300, H=2, dk=128, dv=128, dt=1, chunk=64, ck=P(9), every=64,
           slots=4, ws=P(10), ws_bytes=1 << 30):
    lib.kda_prefill_varlen.argtypes = [ctypes.c_void_p] * 9 + [ctypes.c_int] * 7 + \
        [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t,
         ctypes.c_void_p]
    return lib.kda_prefill_varlen(q, k, v, la, beta, S0, o, Sf, cu, N, T, H, dk, dv, dt, chunk,
                                  ck, every, slots, ws, ws_bytes, None)


def test_varlen_workspace_query(lib):
    f = lib.kda_prefill_varlen_workspace_size
    f.restype = ctypes.c_size_t
    tab = f(3, 300, 64, 128, 128, 1, 64)             # 192 sequence-heads: fused, table only
    assert tab == 256
    assert f(3, 300, 64, 128, 128, 0, 64) == 256     # fp32 path: table only
    few = f(3, 300, 2, 128, 128, 1, 64)              # 6 sequence-heads: records too
    assert few > tab and (few - tab) % (2 * ((300 + 3 * 63) // 64)) == 0
    assert f(0, 300, 2, 128, 128, 1, 64) == 0
    assert f(3, 300, 2, 48, 128, 1, 64) == 0         # unsupported
    # 576 sequence-heads: the split schedule's tables, end states and records
    # (at most 16384 chunk-heads of 72,192 B)
    rec = 16384 * 72192
    big = f(18, 65536, 32, 128, 128, 1, 64)
    assert rec < big < rec + (64 << 20)
    assert f(18, 65536, 32, 128, 128, 0, 64) == 256  # fp32: no split schedule
    # more than 1024 sequences, or 256 heads or more (no sequence can exceed
    # an even share): table only
    assert f(1025, 65536, 32, 128, 128, 1, 64) == (3 * 1025 + 3) * 4 + 255 & ~255
    assert f(2, 65536, 256, 128, 128, 1, 64) == 256


@no_gpu
def test_varlen_rejects(lib):
    assert varlen(lib, N=-1) == INVALID
    assert varlen(lib, T=-1) == INVALID
    assert varlen(lib, dk=48) == UNSUPPORTED
    assert varlen(lib, chunk=128) == UNSUPPORTED
    assert varlen(lib, every=100) == INVALID          # not a multiple of 64
    assert varlen(lib, every=-64) == INVALID
    assert varlen(lib, ck=None) == INVALID            # checkpoints without a buffer
    assert varlen(lib, slots=0) == INVALID
    assert varlen(lib, slots=-1) == INVALID
    assert varlen(lib, cu=None) == INVALID
    assert varlen(lib, cu=P(8, 2)) == INVALID         # cu_seqlens not 4-byte aligned
    for name in ("q", "k", "v", "la", "beta", "o"):
        assert varlen(lib, **{name: None}) == INVALID, name
    for name in ("q", "k", "v", "la", "beta", "S0", "o", "Sf", "ck"):
        assert varlen(lib, **{name: P(11, 4)}) == INVALID, name
    assert varlen(lib, ws=None) == WORKSPACE
    assert varlen(lib, ws_bytes=16) == WORKSPACE
    assert varlen(lib, ws=P(10, 16)) == INVALID       # not 256-byte aligned
    assert varlen(lib, o=P(8)) == INVALID             # o overlapping cu_seqlens
    assert varlen(lib, ck=P(5, 256)) == INVALID       # checkpoints overlapping S0
    assert varlen(lib, ck=P(7)) == INVALID            # checkpoints overlapping S_final
    assert varlen(lib, ws=P(9)) == INVALID            # workspace overlapping checkpoints
    assert varlen(lib, Sf=P(5, 256)) == INVALID       # partial overlap with S0
    assert varlen(lib, N=0) == OK                     # nothing to do
    assert varlen(lib, H=0) == OK


def layer_prefill(lib, opts=None, *, q=P(0), k=P(1), v=P(2), g=P(3), beta=P(4), S0=P(5),
                  o=P(6), Sf=P(7), B=1, T=64, H=2, dk=128, dv=128, dt=1, ws=P(10)):
    return lib.kda_prefill_layer(q, k, v, g, beta, S0, o, Sf, B, T, H, dk, dv, dt, 64,
                                 None if opts is None else ctypes.byref(opts), ws, 1 << 30, None)


def layer_decode(lib, opts=None, *, q=P(0), k=P(1), v=P(2), g=P(3), beta=P(4), S=P(5), o=P(6),
                 B=2, H=2, dk=128, dv=128, dt=1):
    return lib.kda_decode_layer(q, k, v, g, beta, S, o, B, H, dk, dv, dt,
                                None if opts is None else ctypes.byref(opts), None)


@no_gpu
def test_layer_rejects(lib):
    Opts = kda._LayerOpts
    assert ctypes.sizeof(Opts) == 40            # the C struct's layout
    for call in (layer_prefill, layer_decode):
        assert call(lib, Opts(gate=3)) == INVALID            # unknown gate mode
        assert call(lib, Opts(decay_bound=-1.0)) == INVALID
        assert call(lib, Opts(l2_eps=float("nan"))) == INVALID
        assert call(lib, Opts(out_eps=-1e-3)) == INVALID
        assert call(lib, Opts(out_gate=BASE + (8 << 30) + 8)) == INVALID      # z misaligned
        assert call(lib, Opts(out_weight=BASE + (8 << 30) + 2)) == INVALID    # w misaligned
        assert call(lib, Opts(out_gate=BASE + (6 << 30))) == INVALID          # z is o
        assert call(lib, g=None) == INVALID
        assert call(lib, dv=48) == UNSUPPORTED
    assert layer_prefill(lib, Opts(out_weight=BASE + (7 << 30))) == INVALID    # w in S_final
    assert layer_prefill(lib, o=P(3, 1024)) == INVALID       # o inside the gate input
    assert layer_prefill(lib, B=0) == OK
    assert layer_decode(lib, S=P(3, 256)) == INVALID         # S inside the gate input
    assert layer_decode(lib, H=0) == OK
    # the bf16 matrix-core prefill clamps the log-decay into [-5, 0]: a wider
    # bounded gate is refused there, and accepted where the path is exact
    # (other shapes, or the decode step)
    bounded = lambda b: Opts(gate=1, decay_bound=b)
    assert layer_prefill(lib, bounded(5.5)) == UNSUPPORTED
    assert layer_prefill(lib, bounded(5.0), B=0) == OK
    assert layer_prefill(lib, bounded(5.5), B=0) == UNSUPPORTED
    assert layer_prefill(lib, bounded(5.5), dk=64, dv=64, B=0) == OK
    assert layer_decode(lib, bounded(8.0), B=0) == OK


def test_binding_rejects_cpu_tensors():
    import torch
    x = torch.zeros(1, 4, 1, 16)
    with pytest.raises(ValueError):
        kda.kda_prefill_fwd(x, x, x, x, torch.zeros(1, 4, 1))


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    # no fallback: without the built HIP library every entry point raises
    import gated_delta_rule_22_amd as kda_mod
    monkeypatch.setattr(kda_mod, "_lib", None)
    monkeypatch.setattr(kda_mod, "_LIB_PATH", str(tmp_path / "libkda.so"))
    with pytest.raises(RuntimeError, match="missing"):
        kda_mod.load_library()
    import torch
    with pytest.raises(RuntimeError, match="missing"):
        kda_mod.kda_prefill_workspace_size(1, 64, 2, 128, 128, torch.bfloat16)
