"""Pins of the oracle's RMSNorm backward (oracle.rmsnorm_backward) and of
the block's composed backward (oracle.moe_norm_residual_backward), against
facts that do not come from them: PyTorch's autograd (CPU, float64) of the
normalisation formula and of the whole block with the routes held fixed,
the exact halving of dx when x doubles (eps = 0), and the radial identity
sum_h x_h dx_h = 0 (eps = 0: the output does not change along x)."""
import numpy as np
import pytest

import oracle
import workloads as wk

torch = pytest.importorskip("torch")


def _rng(seed):
    return np.random.default_rng(seed)


def _norm_case(T=7, H=64, seed=0, scale=1.0):
    g = _rng(seed)
    x = (g.standard_normal((T, H)) * scale).astype(np.float32)
    w = (1 + 0.1 * g.standard_normal(H)).astype(np.float32)
    gy = g.standard_normal((T, H))
    return x, w, gy


def test_rmsnorm_backward_vs_autograd():
    x, w, gy = _norm_case()
    for eps in (1e-5, 0.3):
        xt = torch.tensor(x.astype(np.float64), requires_grad=True)
        wt = torch.tensor(w.astype(np.float64), requires_grad=True)
        y = wt * xt * torch.rsqrt((xt ** 2).mean(dim=1, keepdim=True) + eps)
        (y * torch.tensor(gy)).sum().backward()
        r = oracle.rmsnorm_backward(x, w, gy, eps)
        # the oracle takes r and n as the fp32 forward has them (~6e-8 relative)
        for got, ref in ((r["dx"], xt.grad.numpy()), (r["dw"], wt.grad.numpy())):
            assert np.abs(got - ref).max() <= 1e-6 * np.abs(ref).max()


def test_rmsnorm_backward_scaling_and_radial_identity():
    x, w, gy = _norm_case(seed=1)
    a = oracle.rmsnorm_backward(x, w, gy, 0.0)
    b = oracle.rmsnorm_backward(x * np.float32(2), w, gy, 0.0)
    assert np.array_equal(b["dx"] * 2, a["dx"]) and np.array_equal(a["dw"], b["dw"])
    rad = (x.astype(np.float64) * a["dx"]).sum(axis=1)
    assert np.all(np.abs(rad) <= 1e-6 * np.abs(x * a["dx"]).sum(axis=1))


def test_rmsnorm_backward_padding_and_magnitudes():
    x, w, gy = _norm_case(T=6, seed=2)
    pad = np.array([0, 1, 0, 0, 1, 0], np.uint8)
    xp = x.copy()
    xp[pad == 1] = np.nan
    mg = np.abs(gy) * 3
    r = oracle.rmsnorm_backward(xp, w, gy, 1e-5, pad, mg=mg)
    assert np.all(np.isnan(r["dx"][pad == 1])) and np.isfinite(r["dx"][pad == 0]).all()
    c = oracle.rmsnorm_backward(x[pad == 0], w, gy[pad == 0], 1e-5, mg=mg[pad == 0])
    assert np.array_equal(r["dx"][pad == 0], c["dx"]) and np.array_equal(r["dw"], c["dw"])
    # the backward is linear in g: a perturbation |dg| <= mg changes dx and
    # dw by at most the magnitudes
    xr, mr = x[pad == 0], mg[pad == 0]
    for seed in range(5):
        dg = mr * _rng(10 + seed).uniform(-1, 1, mr.shape)
        e = oracle.rmsnorm_backward(xr, w, dg, 1e-5)
        assert np.all(np.abs(e["dx"]) <= c["m_dx"] * (1 + 1e-12))
        assert np.all(np.abs(e["dw"]) <= c["m_dw"] * (1 + 1e-12))


def test_block_backward_vs_autograd():
    # out = h + layer(RMSNorm(h)) in torch float64 with the oracle's routes
    # (computed from its own normalised rows); fp32 layer, so the oracle's
    # fp32 roundings of n, xn, u, g and h are the only differences
    K, eps = 2, 1e-5
    shape = wk.LayerShape(H=64, E=4, K=K, I=32, Is=32, dtype=wk.F32)
    wl = wk.custom(shape, (9,))
    d = wk.make_inputs(wl, 3)
    d["w_router"] = d["w_router"] * np.float32(8)
    nw = wk.make_norm_weight(shape, 3)
    dout = wk.make_dout(wl, 3)
    ob = oracle.moe_norm_residual_backward(d["x"], nw, d["w_router"], d["w13"], d["w2"],
                                           d["ws13"], d["ws2"], dout, K, eps)
    xn = oracle.rmsnorm(d["x"], nw, eps)
    route = oracle.route(xn, d["w_router"], K)
    t = {k: torch.tensor(d[k].astype(np.float64), requires_grad=True)
         for k in ("x", "w_router", "w13", "w2", "ws13", "ws2")}
    nwt = torch.tensor(nw.astype(np.float64), requires_grad=True)
    h = t["x"]
    x = nwt * h * torch.rsqrt((h ** 2).mean(dim=1, keepdim=True) + eps)
    p = torch.softmax(x @ t["w_router"].T, dim=-1)

    def swiglu(xr, w13, w2):
        n = w13.shape[0] // 2
        ug = w13 @ xr
        return w2 @ (torch.nn.functional.silu(ug[n:]) * ug[:n])

    outs = []
    for tt in range(x.shape[0]):
        sel = p[tt, route["idx"][tt]]
        wk_ = sel / sel.sum()
        o = h[tt] + swiglu(x[tt], t["ws13"], t["ws2"])
        for k in range(K):
            e = int(route["idx"][tt, k])
            o = o + wk_[k] * swiglu(x[tt], t["w13"][e], t["w2"][e])
        outs.append(o)
    (torch.stack(outs) * torch.tensor(dout.astype(np.float64))).sum().backward()
    pairs = {"dh": t["x"], "dnorm_weight": nwt, "dw_router": t["w_router"], "dw13": t["w13"],
             "dw2": t["w2"], "dws13": t["ws13"], "dws2": t["ws2"]}
    for k, v in pairs.items():
        ref = v.grad.numpy()
        assert np.abs(ob[k] - ref).max() <= 2e-5 * np.abs(ref).max(), k
