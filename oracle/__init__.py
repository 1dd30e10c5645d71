"""CPU oracle of the routed-expert MoE feed-forward layer (ctypes wrapper).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline may import this package; the product path (moe_decoder_ffn_amd)
never does, and shares no code with it. The arithmetic lives in
moe_oracle.c (steps and citations in its header) and dispatch.py.

Arrays are numpy: bf16 tensors as uint16 bit patterns, fp32 as float32.
"""
import ctypes
import os

import numpy as np

from . import build as _build
from .dispatch import dispatch, valid_tokens  # noqa: F401

F32 = 0
BF16 = 1

_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        lib = ctypes.CDLL(_build.LIB)
        P = ctypes.c_void_p
        i64 = ctypes.c_int64
        i32 = ctypes.c_int
        lib.orc_route.argtypes = [P, i32, P, P, i64, i32, i32, P, i64, P, P, P, P]
        lib.orc_route.restype = None
        lib.orc_moe_rows.argtypes = [P, i32, P, P, P, P, P, P, i64, i32, i32, i64,
                                     i64, P, i64, P, P, P, P, P, P]
        lib.orc_moe_rows.restype = None
        lib.orc_moe_dense_rows.argtypes = [P, i32, P, P, P, P, P, i64, i32, i32,
                                           i64, i64, P, i64, P, P, P]
        lib.orc_moe_dense_rows.restype = None
        lib.orc_moe_backward.argtypes = [P, i32, P, P, P, P, P, P, P, i64, i64, i32, i32, i64,
                                         i64, P, P, P, P, P, P, P, P, P, P, P, P, P, P]
        lib.orc_moe_backward.restype = None
        lib.orc_rmsnorm.argtypes = [P, i32, P, ctypes.c_double, P, i64, i64, P]
        lib.orc_rmsnorm.restype = None
        lib.orc_rmsnorm_backward.argtypes = [P, i32, P, ctypes.c_double, P, i64, i64, P, P, P,
                                             P, P, P]
        lib.orc_rmsnorm_backward.restype = None
        lib.orc_round_bf16_array.argtypes = [P, i64, P]
        lib.orc_round_bf16_array.restype = None
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dtype_of(x):
    if x.dtype == np.uint16:
        return BF16
    if x.dtype == np.float32:
        return F32
    raise TypeError(f"unsupported activation dtype {x.dtype}")


def _rows(rows, T):
    if rows is None:
        rows = np.arange(T, dtype=np.int64)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    if rows.size and (rows.min() < 0 or rows.max() >= T):
        raise IndexError("row out of range")
    return rows


def _check_weights(x, w_router, w13, w2, ws13, ws2, K):
    T, H = x.shape
    E = w_router.shape[0]
    if not (1 <= K <= E <= 1024):
        raise ValueError("need 1 <= K <= E <= 1024")
    assert w_router.shape == (E, H) and w_router.dtype == np.float32
    if w13 is not None:
        I = w13.shape[1] // 2
        Is = ws13.shape[0] // 2
        assert w13.shape == (E, 2 * I, H) and w13.dtype == x.dtype
        assert w2.shape == (E, H, I) and w2.dtype == x.dtype
        assert ws13.shape == (2 * Is, H) and ws13.dtype == x.dtype
        assert ws2.shape == (H, Is) and ws2.dtype == x.dtype
        return T, H, E, I, Is
    return T, H, E, None, None


def route(x, w_router, K, pad_mask=None, rows=None):
    """Steps 1-4 for the given rows (all rows by default).

    Returns dict(logits fp32 [n,E], probs fp32 [n,E], idx int32 [n,K],
    w fp32 [n,K]); padding rows give idx -1, w 0."""
    lib = _load()
    x = np.ascontiguousarray(x)
    w_router = np.ascontiguousarray(w_router, np.float32)
    T, H, E, _, _ = _check_weights(x, w_router, None, None, None, None, K)
    rows = _rows(rows, T)
    n = rows.size
    pad = None if pad_mask is None else np.ascontiguousarray(pad_mask, np.uint8)
    logits = np.zeros((n, E), np.float32)
    probs = np.zeros((n, E), np.float32)
    idx = np.zeros((n, K), np.int32)
    w = np.zeros((n, K), np.float32)
    lib.orc_route(_ptr(x), _dtype_of(x), _ptr(w_router), _ptr(pad), H, E, K,
                  _ptr(rows), n, _ptr(logits), _ptr(probs), _ptr(idx), _ptr(w))
    return {"logits": logits, "probs": probs, "idx": idx, "w": w}


def moe(x, w_router, w13, w2, ws13, ws2, K, pad_mask=None, rows=None,
        idx=None, w=None, out=None):
    """The whole layer for the given rows.

    idx/w ([n,K]) replace the router's choice when given. Returns dict(
    out (dtype [n,H], rows of padding left as in `out` if passed, else 0),
    exact (fp64 [n,H], value before the final rounding; NaN for padding rows),
    idx, w)."""
    lib = _load()
    x = np.ascontiguousarray(x)
    dt = _dtype_of(x)
    w_router = np.ascontiguousarray(w_router, np.float32)
    w13, w2, ws13, ws2 = (np.ascontiguousarray(a) for a in (w13, w2, ws13, ws2))
    T, H, E, I, Is = _check_weights(x, w_router, w13, w2, ws13, ws2, K)
    rows = _rows(rows, T)
    n = rows.size
    pad = None if pad_mask is None else np.ascontiguousarray(pad_mask, np.uint8)
    if idx is not None:
        idx = np.ascontiguousarray(idx, np.int32).reshape(n, K)
        w = np.ascontiguousarray(w, np.float64).reshape(n, K)
        if idx.size and (idx.min() < 0 or idx.max() >= E):
            raise ValueError("route id out of range")
    idx_out = np.zeros((n, K), np.int32)
    w_out = np.zeros((n, K), np.float64)
    exact = np.full((n, H), np.nan, np.float64)
    if out is None:
        out = np.zeros((n, H), x.dtype)
    else:
        assert out.shape == (n, H) and out.dtype == x.dtype and out.flags.c_contiguous
    lib.orc_moe_rows(_ptr(x), dt, _ptr(w_router), _ptr(w13), _ptr(w2), _ptr(ws13),
                     _ptr(ws2), _ptr(pad), H, E, K, I, Is, _ptr(rows), n,
                     _ptr(idx), _ptr(w), _ptr(idx_out), _ptr(w_out), _ptr(exact),
                     _ptr(out))
    return {"out": out, "exact": exact, "idx": idx_out, "w": w_out}


def moe_dense(x, w13, w2, ws13, ws2, idx, w, pad_mask=None, rows=None):
    """Dense brute force: all E experts evaluated, each weighted by its gate
    weight if selected in idx/w and by 0 otherwise, plus the shared expert.
    Returns the fp64 value [n,H] (NaN rows for padding)."""
    lib = _load()
    x = np.ascontiguousarray(x)
    dt = _dtype_of(x)
    w13, w2, ws13, ws2 = (np.ascontiguousarray(a) for a in (w13, w2, ws13, ws2))
    T, H = x.shape
    E = w13.shape[0]
    I = w13.shape[1] // 2
    Is = ws13.shape[0] // 2
    rows = _rows(rows, T)
    n = rows.size
    K = idx.shape[1]
    idx = np.ascontiguousarray(idx, np.int32)
    w = np.ascontiguousarray(w, np.float64)
    pad = None if pad_mask is None else np.ascontiguousarray(pad_mask, np.uint8)
    exact = np.full((n, H), np.nan, np.float64)
    lib.orc_moe_dense_rows(_ptr(x), dt, _ptr(w13), _ptr(w2), _ptr(ws13), _ptr(ws2),
                           _ptr(pad), H, E, K, I, Is, _ptr(rows), n, _ptr(idx),
                           _ptr(w), _ptr(exact))
    return exact


def round_bf16(v):
    """fp64 array -> bf16 bit patterns (nearest, ties to even), as the
    oracle's final output rounding does."""
    lib = _load()
    v = np.ascontiguousarray(v, np.float64)
    out = np.empty(v.shape, np.uint16)
    lib.orc_round_bf16_array(_ptr(v), v.size, _ptr(out))
    return out


def rmsnorm(x, weight, eps=1e-5, pad_mask=None):
    """The block's RMSNorm in front of the layer (moe_oracle.c, orc_rmsnorm):
    x [T,H] and weight [H] in the layer dtype. Padding rows of the result are
    zero (never computed)."""
    lib = _load()
    x = np.ascontiguousarray(x)
    dt = _dtype_of(x)
    weight = np.ascontiguousarray(weight)
    T, H = x.shape
    assert weight.shape == (H,) and weight.dtype == x.dtype
    pad = None if pad_mask is None else np.ascontiguousarray(pad_mask, np.uint8)
    xn = np.zeros_like(x)
    lib.orc_rmsnorm(_ptr(x), dt, _ptr(weight), float(eps), _ptr(pad), T, H, _ptr(xn))
    return xn


def _as_f64(a):
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def moe_norm_residual(h, norm_weight, w_router, w13, w2, ws13, ws2, K, eps=1e-5,
                      pad_mask=None, rows=None, idx=None, w=None):
    """The layer inside its block: out = h + layer(RMSNorm(h)) (model API
    page, HunyuanImage3Block: pre-norm, residual around the experts). The
    layer's fp64 value (before its rounding) plus the residual is rounded once
    to the dtype. Returns dict(out [n,H] (zero rows for padding), exact (fp64,
    NaN rows for padding), xn [T,H], idx, w)."""
    h = np.ascontiguousarray(h)
    xn = rmsnorm(h, norm_weight, eps, pad_mask)
    r = moe(xn, w_router, w13, w2, ws13, ws2, K, pad_mask=pad_mask, rows=rows, idx=idx, w=w)
    rows_ = _rows(rows, h.shape[0])
    exact = r["exact"] + _as_f64(h[rows_])
    fin = np.nan_to_num(exact)
    out = round_bf16(fin) if h.dtype == np.uint16 else fin.astype(np.float32)
    if pad_mask is not None:
        out[np.asarray(pad_mask)[rows_] != 0] = 0
    return {"out": out, "exact": exact, "xn": xn, "idx": r["idx"], "w": r["w"]}


def moe_backward(x, w_router, w13, w2, ws13, ws2, dout, K, pad_mask=None, idx=None, w=None,
                 want=("dx", "dw_router", "dw13", "dw2", "dws13", "dws2"), magnitudes=False):
    """Gradients of L = sum over real rows of dout . out (moe_oracle.c,
    orc_moe_backward), with the routes held fixed. dout has x's shape and
    dtype. idx/w ([T,K]) replace the router's choice when given. Returns
    the requested fp64 arrays: dx [T,H] (NaN rows for padding), dw_router
    [E,H], dw13 [E,2I,H], dw2 [E,H,I], dws13 [2Is,H], dws2 [H,Is]; with
    magnitudes=True also "m_<name>": per element the sum of the absolute
    values of the terms summed into it."""
    lib = _load()
    x = np.ascontiguousarray(x)
    dt = _dtype_of(x)
    dout = np.ascontiguousarray(dout)
    assert dout.shape == x.shape and dout.dtype == x.dtype
    w_router = np.ascontiguousarray(w_router, np.float32)
    w13, w2, ws13, ws2 = (np.ascontiguousarray(a) for a in (w13, w2, ws13, ws2))
    T, H, E, I, Is = _check_weights(x, w_router, w13, w2, ws13, ws2, K)
    pad = None if pad_mask is None else np.ascontiguousarray(pad_mask, np.uint8)
    if idx is not None:
        idx = np.ascontiguousarray(idx, np.int32).reshape(T, K)
        w = np.ascontiguousarray(w, np.float64).reshape(T, K)
    shapes = {"dx": (T, H), "dw_router": (E, H), "dw13": (E, 2 * I, H), "dw2": (E, H, I),
              "dws13": (2 * Is, H), "dws2": (H, Is)}
    outs = {k: (np.full(v, np.nan) if k == "dx" else np.zeros(v)) if k in want else None
            for k, v in shapes.items()}
    mags = {k: (np.full(v, np.nan) if k == "dx" else np.zeros(v))
            if (magnitudes and k in want) else None for k, v in shapes.items()}
    names = ("dx", "dw_router", "dw13", "dw2", "dws13", "dws2")
    lib.orc_moe_backward(_ptr(x), dt, _ptr(w_router), _ptr(w13), _ptr(w2), _ptr(ws13),
                         _ptr(ws2), _ptr(pad), _ptr(dout), T, H, E, K, I, Is, _ptr(idx),
                         _ptr(w), *[_ptr(outs[k]) for k in names], *[_ptr(mags[k]) for k in names])
    res = {k: v for k, v in outs.items() if v is not None}
    res.update({"m_" + k: v for k, v in mags.items() if v is not None})
    return res


def rmsnorm_backward(x, weight, g, eps=1e-5, pad_mask=None, mg=None):
    """Backward of rmsnorm (moe_oracle.c, orc_rmsnorm_backward): g = dL/dxn
    (fp64 [T,H]). Returns dict(dx [T,H] fp64 (NaN rows for padding), dw [H]),
    and with mg (magnitudes of g) also m_dx and m_dw."""
    lib = _load()
    x = np.ascontiguousarray(x)
    dt = _dtype_of(x)
    weight = np.ascontiguousarray(weight)
    T, H = x.shape
    assert weight.shape == (H,) and weight.dtype == x.dtype
    g = np.ascontiguousarray(np.nan_to_num(np.asarray(g, np.float64)))
    assert g.shape == (T, H)
    pad = None if pad_mask is None else np.ascontiguousarray(pad_mask, np.uint8)
    mgc = None if mg is None else np.ascontiguousarray(np.nan_to_num(np.asarray(mg, np.float64)))
    dx = np.full((T, H), np.nan)
    dw = np.zeros(H)
    mdx = np.full((T, H), np.nan) if mg is not None else None
    mdw = np.zeros(H) if mg is not None else None
    lib.orc_rmsnorm_backward(_ptr(x), dt, _ptr(weight), float(eps), _ptr(pad), T, H, _ptr(g),
                             _ptr(mgc), _ptr(dx), _ptr(dw), _ptr(mdx), _ptr(mdw))
    res = {"dx": dx, "dw": dw}
    if mg is not None:
        res.update({"m_dx": mdx, "m_dw": mdw})
    return res


def moe_norm_residual_backward(h, norm_weight, w_router, w13, w2, ws13, ws2, dout, K,
                               eps=1e-5, pad_mask=None, idx=None, w=None, magnitudes=False):
    """Gradients of L = sum over real rows of dout . out for the block's
    out = h + layer(RMSNorm(h)) (routes held fixed): the layer's backward at
    the normalised rows, then RMSNorm's, plus dout through the residual.
    Returns dh [T,H] (NaN rows for padding), dnorm_weight [H], and the layer's
    weight gradients (dw_router, dw13, dw2, dws13, dws2); with magnitudes=True
    also m_<name> for each (m_dh is that of the RMSNorm term: dout is
    exact)."""
    h = np.ascontiguousarray(h)
    xn = rmsnorm(h, norm_weight, eps, pad_mask)
    lb = moe_backward(xn, w_router, w13, w2, ws13, ws2, dout, K, pad_mask=pad_mask, idx=idx,
                      w=w, magnitudes=magnitudes)
    nb = rmsnorm_backward(h, norm_weight, lb["dx"], eps, pad_mask,
                          mg=lb["m_dx"] if magnitudes else None)
    res = {k: v for k, v in lb.items() if k not in ("dx", "m_dx")}
    res["dh"] = _as_f64(np.ascontiguousarray(dout)) + nb["dx"]
    res["dnorm_weight"] = nb["dw"]
    if magnitudes:
        res["m_dh"] = nb["m_dx"]
        res["m_dnorm_weight"] = nb["m_dw"]
    return res

