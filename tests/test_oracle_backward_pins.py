"""Pins of the oracle's backward pass (oracle.moe_backward) against facts
that do not come from it: PyTorch's autograd (CPU, float64) on the same
forward with the routes held fixed, central finite differences of the
oracle's own forward, and invariants (experts never selected get no
gradient, padding rows contribute nothing). Catches: a wrong SiLU'
(sigmoid term dropped), up/gate halves swapped in the gradient, dy not
weighted by w, the renormalisation or softmax backward wrong, transposed
weight gradients, the router term of dx missing."""
import numpy as np
import pytest

import oracle
import workloads as wk

torch = pytest.importorskip("torch")


def _as_f64(a):
    if a.dtype == np.uint16:
        return wk.bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def _case(dtype, T=12, H=64, E=4, K=2, I=32, Is=48, seed=1, rscale=8.0, pad=None):
    shape = wk.LayerShape(H=H, E=E, K=K, I=I, Is=Is, dtype=dtype)
    d = wk.make_inputs(wk.custom(shape, (T,)), seed)
    d["w_router"] = d["w_router"] * np.float32(rscale)
    dout = np.random.default_rng(seed + 50).standard_normal((T, H)).astype(np.float32)
    d["dout"] = wk.f32_to_bf16_bits(dout) if dtype == wk.BF16 else dout
    return d


def _torch_grads(d, K, idx, dtype):
    """The layer's forward in torch float64 with fixed routes; h rounded to
    bf16 with a straight-through estimator for bf16 layers (the oracle's
    stored activation); returns the gradients of sum(out * dout)."""
    t = {k: torch.tensor(_as_f64(d[k]), requires_grad=True)
         for k in ("x", "w13", "w2", "ws13", "ws2")}
    wr = torch.tensor(d["w_router"].astype(np.float64), requires_grad=True)
    dout = torch.tensor(_as_f64(d["dout"]))
    x = t["x"]
    T = x.shape[0]
    I = t["w13"].shape[1] // 2
    Is = t["ws13"].shape[0] // 2

    def swiglu(xr, w13, w2, n):
        ug = w13 @ xr
        u, g = ug[:n], ug[n:]
        h = torch.nn.functional.silu(g) * u
        if dtype == wk.BF16:
            hr = torch.tensor(_as_f64(oracle.round_bf16(h.detach().numpy())))
            h = h + (hr - h).detach()
        return w2 @ h

    p = torch.softmax(x @ wr.T, dim=-1)
    out = []
    for tt in range(T):
        sel = p[tt, idx[tt]]
        w = sel / sel.sum()
        o = swiglu(x[tt], t["ws13"], t["ws2"], Is)
        for k in range(K):
            e = int(idx[tt, k])
            o = o + w[k] * swiglu(x[tt], t["w13"][e], t["w2"][e], I)
        out.append(o)
    loss = (torch.stack(out) * dout).sum()
    loss.backward()
    return {"dx": x.grad.numpy(), "dw_router": wr.grad.numpy(), "dw13": t["w13"].grad.numpy(),
            "dw2": t["w2"].grad.numpy(), "dws13": t["ws13"].grad.numpy(),
            "dws2": t["ws2"].grad.numpy()}


@pytest.mark.parametrize("dtype,rtol", [(wk.F32, 2e-6), (wk.BF16, 2e-6)])
def test_backward_vs_torch_autograd(dtype, rtol):
    # fp32 layers: the oracle's fp32 router values and fp32-rounded h differ
    # from float64 torch by ~1e-7 relative; bf16: the same rounding of h on
    # both sides, so again only the router's fp32 values differ
    K = 2
    d = _case(dtype)
    r = oracle.route(d["x"], d["w_router"], K)
    g = oracle.moe_backward(d["x"], d["w_router"], d["w13"], d["w2"], d["ws13"], d["ws2"],
                            d["dout"], K)
    ref = _torch_grads(d, K, r["idx"], dtype)
    for k, v in ref.items():
        scale = np.abs(v).max()
        assert np.max(np.abs(g[k] - v)) <= rtol * 10 * scale + 1e-12, k


def test_backward_finite_differences():
    # L(theta) = sum(out * dout) from the oracle's fp64 forward value; central
    # differences with steps that keep every route; fp32 rounding of h in the
    # forward bounds the agreement at ~1e-4 relative
    K = 2
    d = _case(wk.F32, T=6, H=64, E=4, K=K, I=32, Is=32, seed=3)
    dout = d["dout"].astype(np.float64)

    def loss(dd):
        r = oracle.moe(dd["x"], dd["w_router"], dd["w13"], dd["w2"], dd["ws13"], dd["ws2"], K)
        return float((r["exact"] * dout).sum()), r["idx"]

    g = oracle.moe_backward(d["x"], d["w_router"], d["w13"], d["w2"], d["ws13"], d["ws2"],
                            d["dout"], K)
    _, idx0 = loss(d)
    rng = np.random.default_rng(7)
    checks = [("x", "dx"), ("w_router", "dw_router"), ("w13", "dw13"), ("w2", "dw2"),
              ("ws13", "dws13"), ("ws2", "dws2")]
    for name, gname in checks:
        # entries whose gradient is at least a fifth of the largest one: the
        # fp32 router and the fp32 rounding of h make the loss noisy at the
        # 1e-7 relative level, which would swamp a tiny derivative
        ga = np.abs(g[gname])
        cand = np.argwhere(ga >= 0.2 * ga.max())
        scale = float(np.sqrt(np.mean(d[name].astype(np.float64) ** 2)))
        for j in rng.choice(len(cand), size=min(4, len(cand)), replace=False):
            pos = tuple(int(c) for c in cand[j])
            v0 = float(d[name][pos])
            step = 1e-2 * max(abs(v0), scale)
            dd = {k: v.copy() for k, v in d.items()}
            dd[name][pos] = v0 + step
            lp, ip = loss(dd)
            dd[name][pos] = v0 - step
            lm, im = loss(dd)
            assert np.array_equal(ip, idx0) and np.array_equal(im, idx0)
            # the perturbed values as fp32 numbers
            hstep = (float(np.float32(v0 + step)) - float(np.float32(v0 - step))) / 2.0
            fd = (lp - lm) / (2.0 * hstep)
            an = g[gname][pos]
            assert abs(fd - an) <= 1e-3 * abs(an), (name, pos, fd, an)


def test_backward_unselected_and_padding():
    # experts that no token selects get zero gradients; padding rows add
    # nothing (the result equals the run on the compacted real rows) and
    # their dx rows are not written
    K = 2
    # 4 real tokens select at most 8 of the 16 experts
    d = _case(wk.BF16, T=6, E=16, K=K, seed=5)
    pad = np.zeros(6, np.uint8)
    pad[[1, 4]] = 1
    d["x"][pad == 1] = wk.BF16_NAN
    g = oracle.moe_backward(d["x"], d["w_router"], d["w13"], d["w2"], d["ws13"], d["ws2"],
                            d["dout"], K, pad_mask=pad)
    r = oracle.route(d["x"], d["w_router"], K, pad_mask=pad)
    used = np.unique(r["idx"][pad == 0])
    gr = np.abs(g["dw_router"]).max()
    assert len(used) < 16
    for e in range(16):
        if e not in used:
            assert np.all(g["dw13"][e] == 0) and np.all(g["dw2"][e] == 0)
            # renormalised top-k weights are a softmax over the selected
            # logits alone, so an expert no token selects gets no router
            # gradient either (up to the fp32 rounding of w against p / S)
            assert np.abs(g["dw_router"][e]).max() <= 1e-6 * gr
    # the same shift invariance: the logit gradient of each token sums to 0
    assert np.abs(g["dw_router"].sum(axis=0)).max() <= 1e-6 * gr
    assert np.all(np.isnan(g["dx"][pad == 1]))
    real = pad == 0
    gc = oracle.moe_backward(d["x"][real], d["w_router"], d["w13"], d["w2"], d["ws13"],
                             d["ws2"], d["dout"][real], K)
    for k in gc:
        a = g[k][real] if k == "dx" else g[k]
        assert np.array_equal(a, gc[k]), k


def test_backward_term_magnitudes():
    # the magnitudes bound the gradients (triangle inequality); with one
    # token every expert-weight gradient element is a single term, so the
    # magnitude equals the gradient's absolute value
    K = 2
    d = _case(wk.F32, T=9, seed=11)
    g = oracle.moe_backward(d["x"], d["w_router"], d["w13"], d["w2"], d["ws13"], d["ws2"],
                            d["dout"], K, magnitudes=True)
    for k in ("dx", "dw_router", "dw13", "dw2", "dws13", "dws2"):
        assert np.all(g["m_" + k] >= np.abs(g[k]) * (1 - 1e-12)), k
        assert np.array_equal(g[k], oracle.moe_backward(
            d["x"], d["w_router"], d["w13"], d["w2"], d["ws13"], d["ws2"], d["dout"], K)[k])
    d1 = _case(wk.F32, T=1, seed=12)
    g1 = oracle.moe_backward(d1["x"], d1["w_router"], d1["w13"], d1["w2"], d1["ws13"],
                             d1["ws2"], d1["dout"], K, magnitudes=True)
    for k in ("dw13", "dw2", "dws13", "dws2"):
        assert np.allclose(g1["m_" + k], np.abs(g1[k]), rtol=1e-12, atol=0), k
