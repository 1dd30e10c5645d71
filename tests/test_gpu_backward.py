"""GPU parity of the layer's backward pass (hi3_moe_backward) against the CPU
oracle's backward (oracle.moe_backward): small cases compared on every
element of every gradient (several GEMM tiles, ragged tails, padding, the
small-batch tile configuration), the full-size workload on sampled rows of
dx, plus invariants and determinism.

Routes: the backward recomputes them; the GPU's routes (hi3_moe_route, the
same kernel) are checked against the oracle's by the forward rules, and the
oracle's backward then runs on the GPU's ids where the K-th and (K+1)-th
logits are within the tie tolerance (both selections are correct there).

Tolerance (parity.check_grad): fp32 layers max |err| <= 1e-5 RMS; bf16
layers per element |err| <= ulp + 3 * 2^-8 * (sum of |terms| summed into the
element, from the oracle), and RMS error <= 5e-3 RMS over each tensor.
The forward's 2e-2 RMS max-error bar does not fit gradients: they are sums
over few rows of heavy-tailed products, whose largest elements sit far
above the tensor's RMS and whose cancelling elements far below their terms.
"""
import sys

import numpy as np
import pytest

import oracle
import workloads as wk

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

from parity import (check_grad, check_grad_chunked, check_routes, to_dev, to_host,  # noqa: E402
                    upload)

NAMES = {"dx": "dx", "dw_router": "dw_router", "dw_up_gate": "dw13", "dw_down": "dw2",
         "dw_shared_up_gate": "dws13", "dw_shared_down": "dws2"}


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def gpu_backward(d, K, pad=None):
    import moe_decoder_ffn_amd as m
    dd = upload(d)
    padd = to_dev(pad) if pad is not None else None
    g = m.moe_backward(dd["x"], dd["w_router"], dd["w13"], dd["w2"], dd["ws13"], dd["ws2"],
                       dd["dout"], K, pad_mask=padd)
    _, idx, w, _ = m.moe_forward(dd["x"], dd["w_router"], dd["w13"], dd["w2"], dd["ws13"],
                                 dd["ws2"], K, pad_mask=padd, return_routes=True)
    torch.cuda.synchronize()
    return {k: to_host(v) for k, v in g.items()}, to_host(idx), to_host(w)


def make_case(dtype, H, E, K, I, Is, seq, plen, seed=7, rscale=5.0, skew=False):
    shape = wk.LayerShape(H=H, E=E, K=K, I=I, Is=Is, dtype=dtype)
    wl = wk.custom(shape, seq, plen, skew=skew)
    d = wk.make_inputs(wl, seed)
    d["w_router"] = d["w_router"] * np.float32(rscale)
    d["dout"] = wk.make_dout(wl, seed)
    pad = d.pop("pad_mask")
    return d, (pad if pad.any() else None)


def check_all(d, K, pad, dtype):
    E = d["w_router"].shape[0]
    g, idx, w = gpu_backward(d, K, pad)
    ref = oracle.route(d["x"], d["w_router"], K, pad_mask=pad)
    near, ref_idx, ref_w = check_routes(idx, w, ref, pad, E, K)
    exp = oracle.moe_backward(d["x"], d["w_router"], d["w13"], d["w2"], d["ws13"], d["ws2"],
                              d["dout"], K, pad_mask=pad, idx=ref_idx, w=ref_w,
                              magnitudes=True)
    valid = np.ones(d["x"].shape[0], bool) if pad is None else pad == 0
    errs = {}
    for k, ok in NAMES.items():
        if k == "dx":
            errs[k] = check_grad(g[k][valid], exp[ok][valid], exp["m_" + ok][valid], dtype, k)
            if pad is not None:
                assert np.all(g[k][~valid] == 0), "padding rows of dx were written"
        else:
            errs[k] = check_grad(g[k], exp[ok], exp["m_" + ok], dtype, k)
    return g, errs, near


SMALL = [
    # name, dtype, H, E, K, I, Is, seq_lens, padded_len
    ("tiny_f32", wk.F32, 256, 8, 2, 128, 128, (64,), None),
    ("f32_ragged_pad", wk.F32, 192, 8, 3, 192, 64, (150, 37), 160),
    ("bf16_tiles", wk.BF16, 512, 8, 2, 256, 192, (700,), None),
    ("bf16_e16_pad", wk.BF16, 256, 16, 4, 320, 128, (300, 129, 7), 300),
    ("bf16_e64_k8_stream", wk.BF16, 512, 64, 8, 128, 256, (600,), None),
    ("bf16_one_token", wk.BF16, 256, 8, 2, 128, 128, (1,), None),
    # H and I not multiples of 256: partial column tiles everywhere
    ("bf16_h320_i192", wk.BF16, 320, 8, 3, 192, 320, (400,), None),
    # 64 experts, top-8, 256 rows per expert: the full-size tile
    # configuration (256-row tiles, split dh tiles, several output tiles per
    # weight gradient)
    ("bf16_e64_k8_default_tiles", wk.BF16, 512, 64, 8, 256, 256, (2048,), None),
]


@pytest.mark.parametrize("name,dtype,H,E,K,I,Is,seq,plen", SMALL)
def test_backward_small_all_elements(name, dtype, H, E, K, I, Is, seq, plen):
    _say(f"[backward] {name}")
    d, pad = make_case(dtype, H, E, K, I, Is, seq, plen)
    g, errs, near = check_all(d, K, pad, dtype)
    _say(f"  max err / RMS: " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()))


def test_backward_skewed_router():
    # the skewed router of the skew_16k workload at a small size: four
    # experts take about half of all routes (reductions several tiles deep),
    # four get almost none
    _say("[backward] skewed router")
    d, pad = make_case(wk.BF16, 512, 16, 4, 256, 256, (1500,), None, rscale=1.0, skew=True)
    g, errs, near = check_all(d, 4, pad, wk.BF16)
    _say("  max err / RMS: " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()))


def test_backward_unused_experts_zero_and_deterministic():
    # 3 tokens over 16 experts with K = 2: at least 10 experts get no row;
    # their weight gradients (and router rows) must be exactly zero; two
    # runs are bit-identical
    _say("[backward] unused experts")
    d, pad = make_case(wk.BF16, 256, 16, 2, 128, 128, (3,), None)
    g1, idx, _ = gpu_backward(d, 2)
    g2, _, _ = gpu_backward(d, 2)
    for k in g1:
        assert np.array_equal(g1[k], g2[k]), k
    used = set(np.unique(idx).tolist())
    assert len(used) <= 6
    for e in range(16):
        if e not in used:
            assert np.all(g1["dw_up_gate"][e] == 0) and np.all(g1["dw_down"][e] == 0)
            assert np.all(g1["dw_router"][e] == 0)


def test_backward_zero_dout_gives_zero():
    _say("[backward] zero dout")
    d, pad = make_case(wk.BF16, 256, 8, 2, 128, 128, (100,), None)
    d["dout"] = np.zeros_like(d["dout"])
    g, _, _ = gpu_backward(d, 2)
    for k, v in g.items():
        assert np.all(v.astype(np.float64) == 0) if v.dtype != np.uint16 else np.all(
            (v & 0x7FFF) == 0), k


def test_backward_outputs_optional():
    # any subset of outputs: the computed ones are bit-identical to a full run
    import moe_decoder_ffn_amd as m
    _say("[backward] optional outputs")
    d, pad = make_case(wk.BF16, 256, 8, 2, 128, 128, (200,), None)
    dd = upload(d)
    full = m.moe_backward(dd["x"], dd["w_router"], dd["w13"], dd["w2"], dd["ws13"], dd["ws2"],
                          dd["dout"], 2)
    for want in (("dx",), ("dw_router",), ("dw_down", "dw_shared_up_gate")):
        part = m.moe_backward(dd["x"], dd["w_router"], dd["w13"], dd["w2"], dd["ws13"],
                              dd["ws2"], dd["dout"], 2, want=want)
        assert set(part) == set(want)
        for k in want:
            assert torch.equal(part[k], full[k]), (want, k)


def test_backward_no_rows_zero_weight_gradients():
    import moe_decoder_ffn_amd as m
    _say("[backward] T = 0")
    # a zero-row view of a real allocation: inputs must not be NULL
    x = torch.zeros((1, 256), dtype=torch.bfloat16, device="cuda")[:0]
    wr = torch.ones((8, 256), dtype=torch.float32, device="cuda")
    w13 = torch.ones((8, 256, 256), dtype=torch.bfloat16, device="cuda")
    w2 = torch.ones((8, 256, 128), dtype=torch.bfloat16, device="cuda")
    ws13 = torch.ones((256, 256), dtype=torch.bfloat16, device="cuda")
    ws2 = torch.ones((256, 128), dtype=torch.bfloat16, device="cuda")
    g = m.moe_backward(x, wr, w13, w2, ws13, ws2, x, 2)
    torch.cuda.synchronize()
    for k, v in g.items():
        if k != "dx":
            assert v.numel() > 0 and bool((v == 0).all()), k


@pytest.mark.parametrize("dtype,seq,plen", [(wk.BF16, (300, 129, 7), 300),
                                             (wk.F32, (150, 37), 160)])
def test_training_pair_bit_identical(dtype, seq, plen):
    # hi3_moe_forward_train + hi3_moe_backward_after_forward give exactly what
    # hi3_moe_forward and hi3_moe_backward give on the same inputs
    import moe_decoder_ffn_amd as m
    _say(f"[backward] training pair {dtype}")
    d, pad = make_case(dtype, 256, 16, 4, 192, 128, seq, plen)
    dd = upload(d)
    padd = to_dev(pad)
    x = dd["x"]
    T, H = x.shape
    E, K, I, Is = 16, 4, 192, 128
    w = (dd["w_router"], dd["w13"], dd["w2"], dd["ws13"], dd["ws2"])
    out1, idx1, w1, c1 = m.moe_forward(x, *w, K, pad_mask=padd, return_routes=True)
    g1 = m.moe_backward(x, *w, dd["dout"], K, pad_mask=padd)
    nws = m.hi3_moe_backward_workspace_size(T, H, E, K, I, Is, m.dtype_code(x.dtype))
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    out2 = torch.zeros_like(x)
    idx2 = torch.empty_like(idx1)
    w2 = torch.empty_like(w1)
    c2 = torch.empty_like(c1)
    m.hi3_moe_forward_train(x, *w, padd, K, out2, idx2, w2, c2, ws)
    g2 = {k: torch.zeros_like(v) if k == "dx" else torch.empty_like(v) for k, v in g1.items()}
    m.hi3_moe_backward_after_forward(x, *w, padd, dd["dout"], K, g2["dx"], g2["dw_router"],
                                     g2["dw_up_gate"], g2["dw_down"], g2["dw_shared_up_gate"],
                                     g2["dw_shared_down"], ws)
    torch.cuda.synchronize()
    for a, b in ((out1, out2), (idx1, idx2), (w1, w2), (c1, c2)):
        assert torch.equal(a, b)
    for k in g1:
        assert torch.equal(g1[k], g2[k]), k


def test_autograd_function_matches_entry_points():
    # MoEFunction: out equals hi3_moe_forward's, and the gradients from
    # torch.autograd equal hi3_moe_backward's, bit for bit; unrequested
    # gradients are not computed
    import moe_decoder_ffn_amd as m
    _say("[backward] autograd function")
    d, pad = make_case(wk.BF16, 256, 16, 4, 192, 128, (300, 129, 7), 300)
    dd = upload(d)
    padd = to_dev(pad)
    names = ("x", "w_router", "w13", "w2", "ws13", "ws2")
    leaves = {k: dd[k].clone().requires_grad_(True) for k in names}
    out = m.moe_layer(*(leaves[k] for k in names), 4, padd)
    out.backward(dd["dout"])
    ref_out = m.moe_forward(*(dd[k] for k in names), 4, pad_mask=padd)
    ref = m.moe_backward(*(dd[k] for k in names), dd["dout"], 4, pad_mask=padd)
    torch.cuda.synchronize()
    assert torch.equal(out.detach(), ref_out)
    keys = {"x": "dx", "w_router": "dw_router", "w13": "dw_up_gate", "w2": "dw_down",
            "ws13": "dw_shared_up_gate", "ws2": "dw_shared_down"}
    for k, r in keys.items():
        assert torch.equal(leaves[k].grad, ref[r]), k
    # only x requires a gradient
    x = dd["x"].clone().requires_grad_(True)
    (gx,) = torch.autograd.grad(m.moe_layer(x, *(dd[k] for k in names[1:]), 4, padd),
                                x, dd["dout"])
    assert torch.equal(gx, ref["dx"])


BLOCK = [
    # name, dtype, H, E, K, I, Is, seq_lens, padded_len
    ("block_f32_pad", wk.F32, 192, 8, 3, 192, 64, (150, 37), 160),
    ("block_bf16", wk.BF16, 512, 8, 2, 256, 192, (700,), None),
    ("block_bf16_e16_pad", wk.BF16, 256, 16, 4, 320, 128, (300, 129, 7), 300),
]


@pytest.mark.parametrize("name,dtype,H,E,K,I,Is,seq,plen", BLOCK)
def test_block_backward_all_elements(name, dtype, H, E, K, I, Is, seq, plen):
    # hi3_moe_backward_norm_residual against oracle.moe_norm_residual_backward:
    # dh, the norm weight's gradient and the layer's weight gradients, every
    # element, by the gradient rule
    import moe_decoder_ffn_amd as m
    _say(f"[backward] {name}")
    d, pad = make_case(dtype, H, E, K, I, Is, seq, plen)
    shape = wk.LayerShape(H=H, E=E, K=K, I=I, Is=Is, dtype=dtype)
    nw = wk.make_norm_weight(shape, 7)
    dd = upload(d)
    padd = to_dev(pad)
    nwd = to_dev(nw)
    w = (dd["w_router"], dd["w13"], dd["w2"], dd["ws13"], dd["ws2"])
    g = m.moe_backward_norm_residual(dd["x"], nwd, *w, dd["dout"], K, pad_mask=padd)
    _, idx, wts, _ = m.moe_forward_norm_residual(dd["x"], nwd, *w, K, pad_mask=padd,
                                                 return_routes=True)
    torch.cuda.synchronize()
    g = {k: to_host(v) for k, v in g.items()}
    idx, wts = to_host(idx), to_host(wts)
    xn = oracle.rmsnorm(d["x"], nw, 1e-5, pad)
    ref = oracle.route(xn, d["w_router"], K, pad_mask=pad)
    near, ref_idx, ref_w = check_routes(idx, wts, ref, pad, E, K)
    exp = oracle.moe_norm_residual_backward(d["x"], nw, d["w_router"], d["w13"], d["w2"],
                                            d["ws13"], d["ws2"], d["dout"], K, 1e-5,
                                            pad_mask=pad, idx=ref_idx, w=ref_w, magnitudes=True)
    valid = np.ones(d["x"].shape[0], bool) if pad is None else pad == 0
    names = {"dh": "dh", "dnorm_weight": "dnorm_weight", "dw_router": "dw_router",
             "dw_up_gate": "dw13", "dw_down": "dw2", "dw_shared_up_gate": "dws13",
             "dw_shared_down": "dws2"}
    errs = {}
    for k, ok in names.items():
        if k == "dh":
            errs[k] = check_grad(g[k][valid], exp[ok][valid], exp["m_" + ok][valid], dtype, k)
            if pad is not None:
                assert np.all(g[k][~valid] == 0), "padding rows of dh were written"
        else:
            errs[k] = check_grad(g[k], exp[ok], exp["m_" + ok], dtype, k)
    _say("  max err / RMS: " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()))


def test_block_backward_layer_grads_match_layer_backward():
    # the block's expert and router weight gradients are the layer's at the
    # normalised rows: bit-identical to hi3_moe_backward on RMSNorm(h)
    import moe_decoder_ffn_amd as m
    _say("[backward] block vs layer at xn")
    d, pad = make_case(wk.BF16, 256, 16, 4, 192, 128, (300, 129, 7), 300)
    shape = wk.LayerShape(H=256, E=16, K=4, I=192, Is=128, dtype=wk.BF16)
    nw = to_dev(wk.make_norm_weight(shape, 7))
    dd = upload(d)
    padd = to_dev(pad)
    w = (dd["w_router"], dd["w13"], dd["w2"], dd["ws13"], dd["ws2"])
    gb = m.moe_backward_norm_residual(dd["x"], nw, *w, dd["dout"], 4, pad_mask=padd)
    xn = torch.zeros_like(dd["x"])
    m.hi3_moe_rmsnorm(dd["x"], nw, 1e-5, padd, xn)
    gl = m.moe_backward(xn, *w, dd["dout"], 4, pad_mask=padd)
    torch.cuda.synchronize()
    for k in ("dw_router", "dw_up_gate", "dw_down", "dw_shared_up_gate", "dw_shared_down"):
        assert torch.equal(gb[k], gl[k]), k


def test_block_autograd_function():
    import moe_decoder_ffn_amd as m
    _say("[backward] block autograd function")
    d, pad = make_case(wk.BF16, 256, 16, 4, 192, 128, (300, 129, 7), 300)
    shape = wk.LayerShape(H=256, E=16, K=4, I=192, Is=128, dtype=wk.BF16)
    nw = to_dev(wk.make_norm_weight(shape, 7))
    dd = upload(d)
    padd = to_dev(pad)
    names = ("x", "w_router", "w13", "w2", "ws13", "ws2")
    leaves = {k: dd[k].clone().requires_grad_(True) for k in names}
    nwl = nw.clone().requires_grad_(True)
    out = m.moe_block(leaves["x"], nwl, *(leaves[k] for k in names[1:]), 4, pad_mask=padd)
    out.backward(dd["dout"])
    ref_out = m.moe_forward_norm_residual(dd["x"], nw, *(dd[k] for k in names[1:]), 4,
                                          pad_mask=padd)
    ref = m.moe_backward_norm_residual(dd["x"], nw, *(dd[k] for k in names[1:]), dd["dout"], 4,
                                       pad_mask=padd)
    torch.cuda.synchronize()
    assert torch.equal(out.detach(), ref_out)
    assert torch.equal(leaves["x"].grad, ref["dh"]) and torch.equal(nwl.grad, ref["dnorm_weight"])
    keys = {"w_router": "dw_router", "w13": "dw_up_gate", "w2": "dw_down",
            "ws13": "dw_shared_up_gate", "ws2": "dw_shared_down"}
    for k, r in keys.items():
        assert torch.equal(leaves[k].grad, ref[r]), k


@pytest.mark.parametrize("name", ["image_1024"])
def test_backward_full_size_sampled_rows(name):
    # full size, the launch configuration the benchmark times: dx of sampled
    # rows against the oracle (dx of a row depends on that row alone); every
    # gradient finite; deterministic
    _say(f"[backward] full size {name}")
    wl = wk.workload(name)
    d = wk.make_inputs(wl, 0)
    d["dout"] = wk.make_dout(wl, 0)
    pad = d.pop("pad_mask")
    pad = pad if pad.any() else None
    K, E = wl.shape.K, wl.shape.E
    g, idx, w = gpu_backward(d, K, pad)
    ref = oracle.route(d["x"], d["w_router"], K, pad_mask=pad)
    near, ref_idx, ref_w = check_routes(idx, w, ref, pad, E, K)
    for k, v in g.items():
        f = v.astype(np.float64) if v.dtype != np.uint16 else wk.bf16_bits_to_f32(v)
        assert np.isfinite(f).all(), k
    T = d["x"].shape[0]
    rows = np.array([0, 1, T // 2, T - 1])
    sub = {k: d[k][rows] for k in ("x", "dout")}
    exp = oracle.moe_backward(sub["x"], d["w_router"], d["w13"], d["w2"], d["ws13"], d["ws2"],
                              sub["dout"], K, idx=ref_idx[rows], w=ref_w[rows], want=("dx",),
                              magnitudes=True)
    check_grad(g["dx"][rows], exp["dx"], exp["m_dx"], wl.shape.dtype, "dx")
    g2, _, _ = gpu_backward(d, K, pad)
    for k in g:
        assert np.array_equal(g[k], g2[k]), k
    # linear in dout, exactly: doubling dout doubles every product and sum,
    # and rounding commutes with a power-of-two scaling, so every gradient
    # doubles bit for bit (a read of stale or uninitialised memory would not)
    d2 = dict(d)
    d2["dout"] = wk.f32_to_bf16_bits(wk.bf16_bits_to_f32(d["dout"]) * np.float32(2.0))
    g3, _, _ = gpu_backward(d2, K, pad)
    for k in g:
        a = g[k].astype(np.float64) if g[k].dtype != np.uint16 else wk.bf16_bits_to_f32(g[k])
        b = g3[k].astype(np.float64) if g3[k].dtype != np.uint16 else wk.bf16_bits_to_f32(g3[k])
        assert np.array_equal(2 * a, b), k
    # the logit gradient of each token sums to zero (renormalised weights do
    # not change when every selected logit moves together), so the rows of
    # the router's weight gradient cancel up to rounding
    dwr = g["dw_router"].astype(np.float64)
    assert np.abs(dwr.sum(axis=0)).max() <= 1e-3 * np.abs(dwr).sum(axis=0).max()


def test_backward_full_shape_every_element():
    """The full layer shape (H = 4096, E = 64, K = 8, I = I_shared = 3072) on
    a short padded batch, four sequences of 4 real tokens right-padded to 16
    (16 real rows of 64): every element of every gradient, the full-shape
    weight gradients included, against the oracle's backward (about a minute
    of oracle time). Experts that no real row selects must get exactly zero
    gradients; padding rows of dx are never written."""
    _say("[backward] full shape, 16 real rows, every element")
    shape = wk.FULL
    wl = wk.custom(shape, (4, 4, 4, 4), padded_len=16)
    d = wk.make_inputs(wl, 5)
    d["dout"] = wk.make_dout(wl, 5)
    pad = d.pop("pad_mask")
    K, E = shape.K, shape.E
    g, idx, w = gpu_backward(d, K, pad)
    ref = oracle.route(d["x"], d["w_router"], K, pad_mask=pad)
    near, ref_idx, ref_w = check_routes(idx, w, ref, pad, E, K)
    _say("  oracle backward")
    exp = oracle.moe_backward(d["x"], d["w_router"], d["w13"], d["w2"], d["ws13"], d["ws2"],
                              d["dout"], K, pad_mask=pad, idx=ref_idx, w=ref_w, magnitudes=True)
    valid = pad == 0
    errs = {"dx": check_grad(g["dx"][valid], exp["dx"][valid], exp["m_dx"][valid], wk.BF16,
                             "dx")}
    assert np.all(g["dx"][~valid] == 0), "padding rows of dx were written"
    errs["dw_router"] = check_grad(g["dw_router"], exp["dw_router"], exp["m_dw_router"],
                                   wk.BF16, "dw_router")
    for k in ("dw_up_gate", "dw_down", "dw_shared_up_gate", "dw_shared_down"):
        ok = NAMES[k]
        errs[k] = check_grad_chunked(g[k], exp[ok], exp["m_" + ok], wk.BF16, k)
        del exp[ok], exp["m_" + ok]
    used = np.unique(ref_idx[valid])
    unused = np.setdiff1d(np.arange(E), used)
    assert unused.size > 0
    for k in ("dw_up_gate", "dw_down"):
        assert not np.any(g[k][unused]), k
    assert not np.any(g["dw_router"][unused])
    _say(f"  experts used {used.size}, max err / RMS: " +
         ", ".join(f"{k} {v:.2e}" for k, v in errs.items()))


def test_block_backward_and_training_pair_full_size():
    # image_1024: the block backward's dh on sampled rows against the oracle
    # (dh of a row depends on that row alone) and its exact doubling with
    # dout; the training pair bit-identical to the standalone calls
    import moe_decoder_ffn_amd as m
    _say("[backward] full size block + training pair")
    wl = wk.workload("image_1024")
    d = wk.make_inputs(wl, 0)
    d["dout"] = wk.make_dout(wl, 0)
    pad = d.pop("pad_mask")
    pad = pad if pad.any() else None
    sh = wl.shape
    K, E = sh.K, sh.E
    nw = wk.make_norm_weight(sh, 0)
    dd = upload(d)
    nwd = to_dev(nw)
    padd = to_dev(pad) if pad is not None else None
    w = (dd["w_router"], dd["w13"], dd["w2"], dd["ws13"], dd["ws2"])
    gb = m.moe_backward_norm_residual(dd["x"], nwd, *w, dd["dout"], K, pad_mask=padd)
    dout2 = to_dev(wk.f32_to_bf16_bits(wk.bf16_bits_to_f32(d["dout"]) * np.float32(2.0)))
    gb2 = m.moe_backward_norm_residual(dd["x"], nwd, *w, dout2, K, pad_mask=padd)
    _, idx, wts, _ = m.moe_forward_norm_residual(dd["x"], nwd, *w, K, pad_mask=padd,
                                                 return_routes=True)
    torch.cuda.synchronize()
    for k in gb:
        a, b = gb[k].float(), gb2[k].float()
        assert torch.equal(2 * a, b), k
    dh = to_host(gb["dh"])
    idx, wts = to_host(idx), to_host(wts)
    xn = oracle.rmsnorm(d["x"], nw, 1e-5, pad)
    ref = oracle.route(xn, d["w_router"], K, pad_mask=pad)
    near, ref_idx, ref_w = check_routes(idx, wts, ref, pad, E, K)
    T = d["x"].shape[0]
    rows = np.array([0, T // 3, T - 1])
    exp = oracle.moe_norm_residual_backward(d["x"][rows], nw, d["w_router"], d["w13"], d["w2"],
                                            d["ws13"], d["ws2"], d["dout"][rows], K, 1e-5,
                                            idx=ref_idx[rows], w=ref_w[rows], magnitudes=True)
    check_grad(dh[rows], exp["dh"], exp["m_dh"], sh.dtype, "dh")
    # training pair at full size
    x = dd["x"]
    g1 = m.moe_backward(x, *w, dd["dout"], K, pad_mask=padd)
    out1 = m.moe_forward(x, *w, K, pad_mask=padd)
    nws = m.hi3_moe_backward_workspace_size(T, sh.H, E, K, sh.I, sh.Is, m.dtype_code(x.dtype))
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    out2 = torch.zeros_like(x)
    m.hi3_moe_forward_train(x, *w, padd, K, out2, workspace=ws)
    g2 = {k: torch.zeros_like(v) if k == "dx" else torch.empty_like(v) for k, v in g1.items()}
    m.hi3_moe_backward_after_forward(x, *w, padd, dd["dout"], K, g2["dx"], g2["dw_router"],
                                     g2["dw_up_gate"], g2["dw_down"], g2["dw_shared_up_gate"],
                                     g2["dw_shared_down"], ws)
    torch.cuda.synchronize()
    assert torch.equal(out1, out2)
    for k in g1:
        assert torch.equal(g1[k], g2[k]), k

