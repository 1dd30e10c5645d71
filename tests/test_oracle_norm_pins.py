"""Pins of the oracle's block normalisation and residual (oracle.rmsnorm,
oracle.moe_norm_residual) against facts that do not come from the oracle:
numpy float64 formulas, closed forms for constant rows, exact invariants
(power-of-two scaling, zero experts), and the single-expert reduction to
dense MLPs. Each catches a class of mistake: eps dropped or misplaced, sum
instead of mean, weight not applied or indexed by row, the router or the
experts fed the unnormalised rows, the residual dropped or added twice,
padding read."""
import math

import numpy as np
import pytest

import oracle
import workloads as wk


def _as_f64(a):
    if a.dtype == np.uint16:
        return wk.bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def _to_dtype(v, dtype):
    v = np.asarray(v, np.float32)
    return wk.f32_to_bf16_bits(v) if dtype == wk.BF16 else v


def _rows(dtype, T, H, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H)).astype(np.float32) * np.float32(scale)
    return _to_dtype(x, dtype)


def _np_rmsnorm(x64, w64, eps):
    return w64 * x64 / np.sqrt(np.mean(x64 ** 2, axis=1, keepdims=True) + eps)


@pytest.mark.parametrize("dtype,rel", [(wk.F32, 2.0 ** -21), (wk.BF16, 2.0 ** -7)])
def test_rmsnorm_vs_numpy_float64(dtype, rel):
    # fp32: three fp32 roundings at most; bf16: two half-ulp roundings (one
    # ulp of 2^-7 relative) plus the fp32 steps.
    T, H = 40, 320
    x = _rows(dtype, T, H, 0)
    x[1] = _to_dtype(_as_f64(x[1]) * 1e-3, dtype)        # small row: eps matters
    x[2] = _to_dtype(_as_f64(x[2]) * 300.0, dtype)       # large row
    w = _to_dtype(1.0 + 0.3 * np.random.default_rng(1).standard_normal(H), dtype)
    xn = oracle.rmsnorm(x, w, 1e-5)
    ref = _np_rmsnorm(_as_f64(x), _as_f64(w), 1e-5)
    err = np.abs(_as_f64(xn) - ref)
    assert np.all(err <= rel * np.abs(ref) + 1e-30)


@pytest.mark.parametrize("dtype", [wk.F32, wk.BF16])
def test_rmsnorm_constant_rows_closed_form(dtype):
    # A constant row c gives c / sqrt(c^2 + eps) in every element (weight 1).
    # c = 2^-8: c^2 = 2^-16 is comparable to eps = 1e-5, so eps inside the
    # square root, added to the mean, is what sets the value:
    # 2^-8 / sqrt(2^-16 + 1e-5) = 0.7772... -> bf16 0.77734375 (199 / 256);
    # without eps the result would be 1.
    H = 64
    cs = [2.0 ** -8, 1.5, 0.001, 40.0]
    x = _to_dtype(np.array([[c] * H for c in cs]), dtype)
    w = _to_dtype(np.ones(H), dtype)
    xn = _as_f64(oracle.rmsnorm(x, w, 1e-5))
    for i, c in enumerate(cs):
        v = c / math.sqrt(c * c + 1e-5)
        if dtype == wk.BF16:
            # nearest bf16 of v (v in [0.5, 1): spacing 2^-8), ties cannot occur
            v = round(v * 256.0) / 256.0
            assert np.all(xn[i] == v), (c, xn[i][0], v)
        else:
            assert np.all(np.abs(xn[i] - v) <= 2.0 ** -22), (c, xn[i][0], v)
    if dtype == wk.BF16:
        assert xn[0, 0] == 0.77734375


@pytest.mark.parametrize("dtype", [wk.F32, wk.BF16])
def test_rmsnorm_zero_row_is_zero(dtype):
    H = 128
    x = _to_dtype(np.zeros((3, H)), dtype)
    w = _to_dtype(np.ones(H), dtype)
    xn = _as_f64(oracle.rmsnorm(x, w, 1e-5))
    assert np.all(xn == 0.0)


@pytest.mark.parametrize("dtype", [wk.F32, wk.BF16])
def test_rmsnorm_scale_invariance_and_weight(dtype):
    # With eps = 0 a power-of-two scale of the row cancels exactly; a weight
    # of 2 doubles every element exactly; a one-hot weight keeps one column.
    T, H = 12, 192
    x = _rows(dtype, T, H, 4)
    w = _to_dtype(1.0 + 0.2 * np.random.default_rng(5).standard_normal(H), dtype)
    base = oracle.rmsnorm(x, w, 0.0)
    for k in (-3, 5):
        xs = _to_dtype(_as_f64(x) * 2.0 ** k, dtype)
        assert np.array_equal(oracle.rmsnorm(xs, w, 0.0), base)
    ones = _to_dtype(np.ones(H), dtype)
    twos = _to_dtype(np.full(H, 2.0), dtype)
    assert np.array_equal(_as_f64(oracle.rmsnorm(x, twos, 1e-5)),
                          2.0 * _as_f64(oracle.rmsnorm(x, ones, 1e-5)))
    onehot = np.zeros(H)
    onehot[37] = 1.0
    xn = _as_f64(oracle.rmsnorm(x, _to_dtype(onehot, dtype), 1e-5))
    assert np.all(xn[:, np.arange(H) != 37] == 0.0) and np.all(xn[:, 37] != 0.0)


def test_rmsnorm_padding_not_read():
    T, H = 10, 128
    x = _rows(wk.BF16, T, H, 6)
    pad = np.zeros(T, np.uint8)
    pad[[2, 7]] = 1
    x[pad == 1] = wk.BF16_NAN
    w = _to_dtype(np.ones(H), wk.BF16)
    xn = oracle.rmsnorm(x, w, 1e-5, pad)
    assert np.all(xn[pad == 1] == 0)
    assert np.array_equal(xn[pad == 0], oracle.rmsnorm(x[pad == 0], w, 1e-5))


def _norm_case(dtype, T, H, E, K, I, Is, seed, hscale):
    shape = wk.LayerShape(H=H, E=E, K=K, I=I, Is=Is, dtype=dtype)
    d = wk.make_weights(shape, seed)
    h = _rows(dtype, T, H, seed + 100, hscale)
    return d, h, wk.make_norm_weight(shape, seed)


@pytest.mark.parametrize("dtype", [wk.F32, wk.BF16])
def test_zero_experts_leave_the_residual(dtype):
    # All expert weights zero: every SwiGLU output is exactly 0, so the block
    # returns h bit for bit (one residual, nothing else).
    d, h, nw = _norm_case(dtype, 16, 128, 8, 2, 64, 64, 1, 3.0)
    z = {k: np.zeros_like(d[k]) for k in ("w13", "w2", "ws13", "ws2")}
    r = oracle.moe_norm_residual(h, nw, d["w_router"], z["w13"], z["w2"], z["ws13"], z["ws2"], 2)
    assert np.array_equal(r["out"], h)


def _np_swiglu(x64, w13, w2, dtype):
    I = w13.shape[0] // 2
    uv = x64 @ _as_f64(w13).T
    u, g = uv[:, :I], uv[:, I:]
    hh = g / (1.0 + np.exp(-g)) * u
    if dtype == wk.BF16:
        hh = _as_f64(oracle.round_bf16(hh))
    else:
        hh = hh.astype(np.float32).astype(np.float64)
    return hh @ _as_f64(w2).T


@pytest.mark.parametrize("dtype", [wk.F32, wk.BF16])
def test_norm_residual_reduces_to_numpy_mlps(dtype):
    # E = 4, K = 2 with a large router scale and a residual of RMS 5:
    # out = h + sum_k w_k SwiGLU_k(n) + SwiGLU_s(n), n = RMSNorm(h), all in
    # numpy float64 (n taken from the numpy formula, routes from numpy
    # softmax/argsort on the normalised rows). Feeding the router or the
    # experts with h instead of n, or dropping the residual, is far outside
    # the bound.
    T, H, E, K = 24, 128, 4, 2
    d, h, nw = _norm_case(dtype, T, H, E, K, 64, 64, 2, 5.0)
    wr = d["w_router"] * np.float32(8.0)
    r = oracle.moe_norm_residual(h, nw, wr, d["w13"], d["w2"], d["ws13"], d["ws2"], K)
    n64 = _np_rmsnorm(_as_f64(h), _as_f64(nw), 1e-5)
    n64 = _as_f64(_to_dtype(n64, dtype))
    logits = n64 @ wr.astype(np.float64).T
    p = np.exp(logits - logits.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    order = np.argsort(-logits, axis=1, kind="stable")[:, :K]
    moe = _np_swiglu(n64, d["ws13"], d["ws2"], dtype)
    for t in range(T):
        sel = order[t]
        ws = p[t, sel] / p[t, sel].sum()
        for k in range(K):
            moe[t] += ws[k] * _np_swiglu(n64[t:t + 1], d["w13"][sel[k]], d["w2"][sel[k]], dtype)[0]
    ref = _as_f64(h) + moe
    same = np.all(np.sort(r["idx"], 1) == np.sort(order, 1), axis=1)
    assert same.mean() > 0.9
    scale = np.sqrt(np.mean(moe[same] ** 2))
    # n differs from the numpy value by at most one rounding step per element
    assert np.max(np.abs(r["exact"][same] - ref[same])) <= 0.05 * scale
    # and the residual is added exactly once
    assert np.max(np.abs((r["exact"] - _as_f64(h))[same] - moe[same])) <= 0.05 * scale
