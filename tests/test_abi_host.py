"""The C ABI on the host (no GPU needed): the library loads, exports every
function include/hi3_moe.h declares, and rejects bad arguments with the
documented status before enqueuing anything. Only validation paths and
host-only functions are called here; fake device pointers are never
dereferenced because validation fails (or T = 0 returns) first."""
import ctypes
import os
import re
import subprocess

import pytest

import moe_decoder_ffn_amd as m

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hi3_moe.h")

# fake, 256-byte aligned "device" addresses; never dereferenced
P = 0x7F0000000000
UNALIGNED = P + 8


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\**\s*(hi3_moe_\w+)\s*\(", text, re.M)))


def test_header_declarations_match_binding():
    decl = declared_functions()
    assert decl == sorted(m.EXPORTED)


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", m.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (hi3_moe_\w+)", out))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(m.lib, name)


def test_status_strings_and_stage_names():
    for s in (m.HI3_OK, m.HI3_E_NULL, m.HI3_E_SHAPE, m.HI3_E_UNSUPPORTED,
              m.HI3_E_WORKSPACE, m.HI3_E_HIP):
        assert m.hi3_moe_status_string(s) not in ("", "unknown status")
    assert m.hi3_moe_status_string(12345) == "unknown status"
    names = [m.hi3_moe_stage_name(i) for i in range(m.HI3_NUM_STAGES)]
    assert len(set(names)) == m.HI3_NUM_STAGES and "?" not in names
    assert m.hi3_moe_stage_name(m.HI3_NUM_STAGES) == "?"


def test_workspace_size():
    ws = m.hi3_moe_workspace_size
    full = ws(4131, 4096, 64, 8, 3072, 3072, m.HI3_BF16)
    route = ws(4131, 4096, 64, 8, 0, 0, m.HI3_BF16)
    assert 0 < route < full
    # buffers that dominate at full size: SwiGLU activations and fp32 expert
    # outputs (routed and shared); token rows are read from x in place
    TK = 4131 * 8
    big = TK * 3072 * 2 + 4131 * 3072 * 2 + TK * 4096 * 4 + 4131 * 4096 * 4
    assert big <= full <= big + 64 * 2 ** 20
    assert ws(0, 4096, 64, 8, 3072, 3072, m.HI3_BF16) == 0
    for bad in [(-1, 4096, 64, 8, 3072, 3072, 1), (10, 4096, 64, 65, 3072, 3072, 1),
                (10, 4096, 65, 8, 3072, 3072, 1), (10, 4000, 64, 8, 3072, 3072, 1),
                (10, 4096, 64, 8, 3000, 3072, 1), (10, 4096, 64, 8, 3072, 3072, 2)]:
        assert ws(*bad) == 0, bad
    # monotone in T
    assert ws(100, 256, 8, 2, 128, 128, 0) < ws(1000, 256, 8, 2, 128, 128, 0)


def _fwd(**kw):
    a = dict(x=P, wr=P, w13=P, w2=P, ws13=P, ws2=P, pad=None, T=64, H=256, E=8, K=2, I=128,
             Is=128, dt=m.HI3_F32, out=P, idx=None, w=None, cnt=None, ws=P,
             wsb=1 << 40, stream=None)
    a.update(kw)
    return m.lib.hi3_moe_forward(a["x"], a["wr"], a["w13"], a["w2"], a["ws13"], a["ws2"],
                                 a["pad"], a["T"], a["H"], a["E"], a["K"], a["I"], a["Is"],
                                 a["dt"], a["out"], a["idx"], a["w"], a["cnt"], a["ws"],
                                 a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), m.HI3_E_NULL),
    (dict(wr=None), m.HI3_E_NULL),
    (dict(w13=None), m.HI3_E_NULL),
    (dict(w2=None), m.HI3_E_NULL),
    (dict(ws13=None), m.HI3_E_NULL),
    (dict(ws2=None), m.HI3_E_NULL),
    (dict(out=None), m.HI3_E_NULL),
    (dict(ws=None), m.HI3_E_NULL),
    (dict(T=-1), m.HI3_E_SHAPE),
    (dict(H=0), m.HI3_E_SHAPE),
    (dict(E=0), m.HI3_E_SHAPE),
    (dict(K=0), m.HI3_E_SHAPE),
    (dict(K=9), m.HI3_E_SHAPE),
    (dict(I=0), m.HI3_E_SHAPE),
    (dict(Is=-64), m.HI3_E_SHAPE),
    (dict(dt=7), m.HI3_E_UNSUPPORTED),
    (dict(E=65, K=8), m.HI3_E_UNSUPPORTED),
    (dict(H=250), m.HI3_E_UNSUPPORTED),
    (dict(I=100), m.HI3_E_UNSUPPORTED),
    (dict(Is=96), m.HI3_E_UNSUPPORTED),
    (dict(T=1 << 29, K=8, E=8), m.HI3_E_UNSUPPORTED),
    (dict(x=UNALIGNED), m.HI3_E_UNSUPPORTED),
    (dict(out=UNALIGNED), m.HI3_E_UNSUPPORTED),
    (dict(pad=UNALIGNED), m.HI3_E_UNSUPPORTED),
    (dict(idx=UNALIGNED), m.HI3_E_UNSUPPORTED),
    (dict(wsb=1000), m.HI3_E_WORKSPACE),
    (dict(T=0), m.HI3_OK),
    (dict(T=0, ws=None), m.HI3_OK),
])
def test_forward_validation(kw, status):
    assert _fwd(**kw) == status


def test_forward_workspace_boundary():
    need = m.hi3_moe_workspace_size(64, 256, 8, 2, 128, 128, m.HI3_F32)
    assert _fwd(wsb=need - 1) == m.HI3_E_WORKSPACE


def test_route_and_dispatch_validation():
    r = m.lib.hi3_moe_route
    need = m.hi3_moe_workspace_size(64, 256, 8, 2, 0, 0, m.HI3_BF16)
    assert r(None, P, None, 64, 256, 8, 2, 1, P, P, None, P, need, None) == m.HI3_E_NULL
    assert r(P, P, None, 64, 256, 8, 2, 1, None, P, None, P, need, None) == m.HI3_E_NULL
    assert r(P, P, None, 64, 256, 8, 9, 1, P, P, None, P, need, None) == m.HI3_E_SHAPE
    assert r(P, P, None, 64, 256, 8, 2, 3, P, P, None, P, need, None) == m.HI3_E_UNSUPPORTED
    assert r(P, P, None, 64, 256, 8, 2, 1, P, P, None, P, need - 1, None) == m.HI3_E_WORKSPACE
    assert r(P, P, None, 64, 256, 8, 2, 1, P, P, UNALIGNED, P, need, None) == m.HI3_E_UNSUPPORTED
    assert r(P, P, None, 0, 256, 8, 2, 1, P, P, None, None, 0, None) == m.HI3_OK
    d = m.lib.hi3_moe_dispatch
    assert d(None, None, P, 64, 256, 8, 2, 1, P, P, P, None, P, need, None) == m.HI3_E_NULL
    assert d(P, None, None, 64, 256, 8, 2, 1, P, P, P, P, P, need, None) == m.HI3_E_NULL
    assert d(P, None, P, 64, 256, 8, 2, 1, P, P, P, None, P, need - 1, None) == m.HI3_E_WORKSPACE
    assert d(P, None, P, 64, 256, 8, 0, 1, P, P, P, None, P, need, None) == m.HI3_E_SHAPE
    assert d(P, None, P, 0, 256, 8, 2, 1, P, P, P, None, None, 0, None) == m.HI3_OK


def test_instrumented_requires_events():
    f = m.lib.hi3_moe_forward_instrumented
    args = [P, P, P, P, P, P, None, 64, 256, 8, 2, 128, 128, 0, P, None, None, None, P,
            1 << 40, None, None]
    assert f(*args, None) == m.HI3_E_NULL


def _fwd_overlap(side, **kw):
    a = dict(x=P, wr=P, w13=P, w2=P, ws13=P, ws2=P, pad=None, T=64, H=256, E=8, K=2, I=128,
             Is=128, dt=m.HI3_BF16, out=P, idx=None, w=None, cnt=None, ws=P,
             wsb=1 << 40, stream=None)
    a.update(kw)
    return m.lib.hi3_moe_forward_overlap(a["x"], a["wr"], a["w13"], a["w2"], a["ws13"],
                                         a["ws2"], a["pad"], a["T"], a["H"], a["E"], a["K"],
                                         a["I"], a["Is"], a["dt"], a["out"], a["idx"], a["w"],
                                         a["cnt"], a["ws"], a["wsb"], a["stream"], side)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), m.HI3_E_NULL),
    (dict(ws2=None), m.HI3_E_NULL),
    (dict(K=9), m.HI3_E_SHAPE),
    (dict(H=250), m.HI3_E_UNSUPPORTED),
    (dict(out=UNALIGNED), m.HI3_E_UNSUPPORTED),
    (dict(wsb=1000), m.HI3_E_WORKSPACE),
    (dict(T=0, ws=None), m.HI3_OK),
])
def test_forward_overlap_validation(kw, status):
    # validation comes before any stream or event is touched: a bogus side
    # stream handle is never used on these paths
    assert _fwd_overlap(P, **kw) == status
    assert _fwd_overlap(None, **kw) == status


def test_no_global_state_in_library_source():
    # the host side keeps nothing between calls: no static streams, events or
    # mutexes (the side stream is the caller's, its events live for one call)
    src = open(os.path.join(ROOT, "moe_decoder_ffn_amd", "csrc", "hi3_moe.cpp")).read()
    for word in ("std::mutex", "static hipStream_t", "static hipEvent_t", "g_side",
                 "hipStreamCreate"):
        assert word not in src, word


def test_shared_on_side_query():
    q = m.hi3_moe_forward_shared_on_side
    # bf16 and no padding mask, whatever the tile plan
    assert q(4131, 4096, 64, 8, 3072, 3072, 1, False)
    assert q(700, 512, 8, 2, 256, 192, 1, False)
    assert q(512, 4096, 64, 8, 3072, 3072, 1, False)        # few rows: streaming tiles
    assert q(1, 4096, 64, 8, 3072, 3072, 1, False)
    assert not q(4131, 4096, 64, 8, 3072, 3072, 1, True)    # padding mask
    assert not q(4131, 4096, 64, 8, 3072, 3072, 0, False)   # fp32
    assert not q(0, 4096, 64, 8, 3072, 3072, 1, False)      # no rows
    assert not q(4131, 4096, 64, 8, 3072, 0, 1, False)      # rejected sizes
    assert not q(4131, 4100, 64, 8, 3072, 3072, 1, False)


def test_package_has_no_fallback():
    # the binding calls the library for everything; nothing under oracle/ is
    # imported by the product package
    import sys
    import importlib
    src = open(os.path.join(ROOT, "moe_decoder_ffn_amd", "__init__.py")).read()
    assert "oracle" not in src.replace("no fallback", "")
    assert "numpy" not in src


def test_rmsnorm_validation():
    f = m.lib.hi3_moe_rmsnorm
    assert f(None, P, 1e-5, None, 64, 256, 1, P, None) == m.HI3_E_NULL
    assert f(P, None, 1e-5, None, 64, 256, 1, P, None) == m.HI3_E_NULL
    assert f(P, P, 1e-5, None, 64, 256, 1, None, None) == m.HI3_E_NULL
    assert f(P, P, 1e-5, None, -1, 256, 1, P, None) == m.HI3_E_SHAPE
    assert f(P, P, 1e-5, None, 64, 0, 1, P, None) == m.HI3_E_SHAPE
    assert f(P, P, 1e-5, None, 64, 250, 1, P, None) == m.HI3_E_UNSUPPORTED
    assert f(P, P, 1e-5, None, 64, 256, 2, P, None) == m.HI3_E_UNSUPPORTED
    assert f(P, P, -1.0, None, 64, 256, 1, P, None) == m.HI3_E_UNSUPPORTED
    assert f(P, P, float("nan"), None, 64, 256, 1, P, None) == m.HI3_E_UNSUPPORTED
    assert f(P, P, float("inf"), None, 64, 256, 1, P, None) == m.HI3_E_UNSUPPORTED
    assert f(UNALIGNED, P, 1e-5, None, 64, 256, 1, P, None) == m.HI3_E_UNSUPPORTED
    assert f(P, P, 1e-5, None, 0, 256, 1, P, None) == m.HI3_OK


def _fwd_nr(**kw):
    a = dict(h=P, nw=P, eps=1e-5, wr=P, w13=P, w2=P, ws13=P, ws2=P, pad=None, T=64, H=256,
             E=8, K=2, I=128, Is=128, dt=m.HI3_BF16, out=P, idx=None, w=None, cnt=None, ws=P,
             wsb=1 << 40, stream=None)
    a.update(kw)
    return m.lib.hi3_moe_forward_norm_residual(
        a["h"], a["nw"], a["eps"], a["wr"], a["w13"], a["w2"], a["ws13"], a["ws2"], a["pad"],
        a["T"], a["H"], a["E"], a["K"], a["I"], a["Is"], a["dt"], a["out"], a["idx"], a["w"],
        a["cnt"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(h=None), m.HI3_E_NULL),
    (dict(nw=None), m.HI3_E_NULL),
    (dict(out=None), m.HI3_E_NULL),
    (dict(K=9), m.HI3_E_SHAPE),
    (dict(eps=-1e-5), m.HI3_E_UNSUPPORTED),
    (dict(eps=float("nan")), m.HI3_E_UNSUPPORTED),
    (dict(nw=UNALIGNED), m.HI3_E_UNSUPPORTED),
    (dict(wsb=1000), m.HI3_E_WORKSPACE),
    (dict(T=0), m.HI3_OK),
])
def test_forward_norm_residual_validation(kw, status):
    assert _fwd_nr(**kw) == status


def _bwd(**kw):
    a = dict(x=P, wr=P, w13=P, w2=P, ws13=P, ws2=P, pad=None, dout=P, T=64, H=256, E=8, K=2,
             I=128, Is=128, dt=m.HI3_BF16, dx=P, dwr=P, dw13=P, dw2=P, dws13=P, dws2=P, ws=P,
             wsb=1 << 40, stream=None)
    a.update(kw)
    return m.lib.hi3_moe_backward(
        a["x"], a["wr"], a["w13"], a["w2"], a["ws13"], a["ws2"], a["pad"], a["dout"], a["T"],
        a["H"], a["E"], a["K"], a["I"], a["Is"], a["dt"], a["dx"], a["dwr"], a["dw13"],
        a["dw2"], a["dws13"], a["dws2"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), m.HI3_E_NULL),
    (dict(wr=None), m.HI3_E_NULL),
    (dict(w13=None), m.HI3_E_NULL),
    (dict(w2=None), m.HI3_E_NULL),
    (dict(ws13=None), m.HI3_E_NULL),
    (dict(ws2=None), m.HI3_E_NULL),
    (dict(dout=None), m.HI3_E_NULL),
    (dict(ws=None), m.HI3_E_NULL),
    (dict(T=-1), m.HI3_E_SHAPE),
    (dict(K=9), m.HI3_E_SHAPE),
    (dict(I=0), m.HI3_E_SHAPE),
    (dict(dt=2), m.HI3_E_UNSUPPORTED),
    (dict(E=65, K=8), m.HI3_E_UNSUPPORTED),
    (dict(H=250), m.HI3_E_UNSUPPORTED),
    (dict(Is=96), m.HI3_E_UNSUPPORTED),
    (dict(dout=UNALIGNED), m.HI3_E_UNSUPPORTED),
    (dict(dx=UNALIGNED), m.HI3_E_UNSUPPORTED),
    (dict(dw13=UNALIGNED), m.HI3_E_UNSUPPORTED),
    (dict(wsb=1000), m.HI3_E_WORKSPACE),
    # no rows and no weight gradient requested: nothing to enqueue
    (dict(T=0, ws=None, dwr=None, dw13=None, dw2=None, dws13=None, dws2=None), m.HI3_OK),
    (dict(T=0, x=None, dout=None, ws=None, dwr=None, dw13=None, dw2=None, dws13=None,
          dws2=None), m.HI3_OK),
])
def test_backward_validation(kw, status):
    assert _bwd(**kw) == status


def test_backward_workspace_size_and_stage_names():
    bws = m.hi3_moe_backward_workspace_size
    need = bws(64, 256, 8, 2, 128, 128, m.HI3_BF16)
    assert need > m.hi3_moe_workspace_size(64, 256, 8, 2, 128, 128, m.HI3_BF16)
    assert _bwd(wsb=need - 1) == m.HI3_E_WORKSPACE
    assert bws(0, 256, 8, 2, 128, 128, 1) == 0
    assert bws(64, 256, 8, 2, 0, 128, 1) == 0
    # dominant buffers at full size: fp32 u, g and dx by slot, then the
    # bf16 slot copies of x, w dout and [du; dg]
    T, TK = 4131, 4131 * 8
    big = TK * 6144 * 4 + TK * 4096 * 4 + TK * 4096 * 2 * 2 + TK * 6144 * 2 + TK * 3072 * 2
    full = bws(T, 4096, 64, 8, 3072, 3072, m.HI3_BF16)
    assert big <= full <= big + 512 * 2 ** 20
    names = [m.hi3_moe_backward_stage_name(i) for i in range(m.HI3_NUM_BWD_STAGES)]
    assert len(set(names)) == m.HI3_NUM_BWD_STAGES and "?" not in names
    assert m.hi3_moe_backward_stage_name(m.HI3_NUM_BWD_STAGES) == "?"
    f = m.lib.hi3_moe_backward_instrumented
    args = [P, P, P, P, P, P, None, P, 64, 256, 8, 2, 128, 128, 1, P, P, P, P, P, P, P,
            1 << 40, None]
    assert f(*args, None) == m.HI3_E_NULL


def test_training_pair_validation():
    need_b = m.hi3_moe_backward_workspace_size(64, 256, 8, 2, 128, 128, m.HI3_BF16)
    need_f = m.hi3_moe_workspace_size(64, 256, 8, 2, 128, 128, m.HI3_BF16)
    assert need_f < need_b
    f = m.lib.hi3_moe_forward_train
    args = [P, P, P, P, P, P, None, 64, 256, 8, 2, 128, 128, 1, P, None, None, None, P]
    # the forward's own workspace is too small: the backward's layout is needed
    assert f(*args, need_f, None) == m.HI3_E_WORKSPACE
    assert f(*args, need_b - 1, None) == m.HI3_E_WORKSPACE
    bad = list(args)
    bad[0] = None
    assert f(*bad, need_b, None) == m.HI3_E_NULL
    g = m.lib.hi3_moe_backward_after_forward
    bargs = [P, P, P, P, P, P, None, P, 64, 256, 8, 2, 128, 128, 1, P, P, P, P, P, P, P]
    assert g(*bargs, need_b - 1, None) == m.HI3_E_WORKSPACE
    bad = list(bargs)
    bad[7] = None
    assert g(*bad, need_b, None) == m.HI3_E_NULL


def test_backward_norm_residual_validation():
    f = m.lib.hi3_moe_backward_norm_residual
    need = m.hi3_moe_backward_workspace_size(64, 256, 8, 2, 128, 128, m.HI3_BF16)

    def call(**kw):
        a = dict(h=P, nw=P, eps=1e-5, dout=P, T=64, dh=P, dnw=P, ws=P, wsb=need)
        a.update(kw)
        return f(a["h"], a["nw"], a["eps"], P, P, P, P, P, None, a["dout"], a["T"], 256, 8, 2,
                 128, 128, 1, a["dh"], a["dnw"], P, P, P, P, P, a["ws"], a["wsb"], None)

    assert call(nw=None) == m.HI3_E_NULL
    assert call(h=None) == m.HI3_E_NULL
    assert call(eps=-1.0) == m.HI3_E_UNSUPPORTED
    assert call(eps=float("nan")) == m.HI3_E_UNSUPPORTED
    assert call(dnw=UNALIGNED) == m.HI3_E_UNSUPPORTED
    assert call(wsb=need - 1) == m.HI3_E_WORKSPACE


def test_probe_validation():
    f = m.lib.hi3_moe_probe_mfma_bf16
    assert f(None, P, 1, 1, None) == m.HI3_E_NULL
    assert f(P, None, 1, 1, None) == m.HI3_E_NULL
    assert f(P, P, 0, 1, None) == m.HI3_E_SHAPE
    assert f(P, P, 1, 0, None) == m.HI3_E_SHAPE
    assert f(UNALIGNED, P, 1, 1, None) == m.HI3_E_UNSUPPORTED


def test_noalloc_validation():
    # checked on the host before any HIP call (no GPU here)
    f = m.lib.hi3_moe_forward_noalloc
    big = (700, 4096, 64, 8, 3072, 3072, m.HI3_BF16)    # more than the scratch holds
    small = (64, 256, 8, 2, 128, 128, m.HI3_BF16)

    def call(sz, x=P, out=P, idx=None, T=None):
        sz = list(sz)
        if T is not None:
            sz[0] = T
        return f(x, P, P, P, P, P, None, *sz, out, idx, None, None, None)

    assert m.hi3_moe_workspace_size(*big) > m.HI3_NOALLOC_SCRATCH_BYTES
    assert call(big) == m.HI3_E_SCRATCH
    assert call(small, x=None) == m.HI3_E_NULL
    assert call(small, out=None) == m.HI3_E_NULL
    assert call(small, idx=UNALIGNED) == m.HI3_E_UNSUPPORTED
    assert call(small, T=-1) == m.HI3_E_SHAPE
    assert call(small, T=0) == m.HI3_OK
    assert m.hi3_moe_status_string(m.HI3_E_SCRATCH) != "unknown status"
