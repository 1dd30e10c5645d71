"""GPU parity of the block's RMSNorm (hi3_moe_rmsnorm, bit for bit: its
rounded rows decide the router's inputs) and of the layer inside its block,
out = h + layer(RMSNorm(h)) (hi3_moe_forward_norm_residual), against the CPU
oracle (oracle.rmsnorm, oracle.moe_norm_residual) under the same rules as
the plain layer: routes by the logit-gap rule, outputs within the dtype's
bar of the oracle's fp64 value."""
import sys

import numpy as np
import pytest

import oracle
import workloads as wk

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

from parity import as_f64, check_output, check_routes, to_dev, to_host, upload  # noqa: E402


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _case(dtype, H, E, K, I, Is, seq, plen, seed, hscale, router_scale=5.0):
    shape = wk.LayerShape(H=H, E=E, K=K, I=I, Is=Is, dtype=dtype)
    wl = wk.custom(shape, seq, plen)
    d = wk.make_inputs(wl, seed)
    d["w_router"] = d["w_router"] * np.float32(router_scale)
    if hscale != 1.0:
        x = as_f64(d["x"]) * hscale
        d["x"] = wk.f32_to_bf16_bits(x.astype(np.float32)) if dtype == wk.BF16 else \
            x.astype(np.float32)
    d["norm_w"] = wk.make_norm_weight(shape, seed)
    pad = d["pad_mask"] if wl.T != wl.T_valid else None
    if pad is not None:
        d["x"][pad == 1] = wk.BF16_NAN if dtype == wk.BF16 else np.nan
    return d, pad


def _gpu_rmsnorm(d, pad, inplace=False):
    import moe_decoder_ffn_amd as m
    x = to_dev(d["x"])
    xn = x if inplace else torch.zeros_like(x)
    m.hi3_moe_rmsnorm(x, to_dev(d["norm_w"]), 1e-5, to_dev(pad), xn)
    torch.cuda.synchronize()
    return to_host(xn)


@pytest.mark.parametrize("dtype", [wk.F32, wk.BF16])
@pytest.mark.parametrize("inplace", [False, True])
@pytest.mark.parametrize("H", [512, 8192, 16384])
def test_rmsnorm_bit_exact(dtype, inplace, H):
    # H = 512 and 8192 keep the row in registers (8 or 16 chunks per lane for
    # bf16), 16384 (and 8192 in fp32) take the two-pass loop
    _say(f"[norm] rmsnorm dtype={dtype} inplace={inplace} H={H}")
    d, pad = _case(dtype, H, 8, 2, 64, 64, (300, 41), 300, 3, 1.0)
    # rows at very different scales, and one all-zero row
    x = as_f64(d["x"])
    x[1] *= 1e-3
    x[2] *= 500.0
    x[3] = 0.0
    d["x"] = wk.f32_to_bf16_bits(x.astype(np.float32)) if dtype == wk.BF16 else \
        x.astype(np.float32)
    d["x"][pad == 1] = wk.BF16_NAN if dtype == wk.BF16 else np.nan
    got = _gpu_rmsnorm(d, pad, inplace)
    ref = oracle.rmsnorm(d["x"], d["norm_w"], 1e-5, pad)
    real = pad == 0
    assert np.array_equal(got[real], ref[real])
    if not inplace:
        assert np.all(got[~real] == 0)


def test_rmsnorm_bit_exact_full_size():
    _say("[norm] rmsnorm full size image_1024")
    wl = wk.workload("image_1024", 0)
    x, pad = wk.make_x(wl, 0)
    d = {"x": x, "norm_w": wk.make_norm_weight(wl.shape, 0)}
    got = _gpu_rmsnorm(d, pad if pad.any() else None)
    ref = oracle.rmsnorm(x, d["norm_w"], 1e-5, pad if pad.any() else None)
    assert np.array_equal(got, ref)


def _gpu_forward_nr(dd, K, pad, sentinel=None, inplace=False):
    import moe_decoder_ffn_amd as m
    h = dd["x"]
    if inplace:
        out = h.clone()
        hin = out
    else:
        hin = h
        out = torch.zeros_like(h) if sentinel is None else torch.full_like(h, sentinel)
    out, idx, w, cnt = m.moe_forward_norm_residual(
        hin, dd["norm_w"], dd["w_router"], dd["w13"], dd["w2"], dd["ws13"], dd["ws2"], K,
        pad_mask=to_dev(pad), out=out, return_routes=True)
    torch.cuda.synchronize()
    return to_host(out), to_host(idx), to_host(w), to_host(cnt)


def _check_nr(d, K, pad, out, idx, w, cnt, rows=None):
    E = d["w_router"].shape[0]
    dtype = wk.BF16 if d["x"].dtype == np.uint16 else wk.F32
    xn = oracle.rmsnorm(d["x"], d["norm_w"], 1e-5, pad)
    ref = oracle.route(xn, d["w_router"], K, pad_mask=pad)
    near, ref_idx, ref_w = check_routes(idx, w, ref, pad, E, K)
    assert np.array_equal(cnt, np.bincount(idx[idx >= 0], minlength=E))
    valid = np.ones(len(idx), bool) if pad is None else pad == 0
    if rows is None:
        rows = np.nonzero(valid)[0]
    r = oracle.moe_norm_residual(d["x"], d["norm_w"], d["w_router"], d["w13"], d["w2"],
                                 d["ws13"], d["ws2"], K, pad_mask=pad, rows=rows,
                                 idx=ref_idx[rows], w=ref_w[rows])
    # the layer's part alone, for the size of the bar
    moe_part = r["exact"] - as_f64(d["x"][rows])
    rel = check_output(out[rows], r["exact"], dtype)
    return rel, float(np.sqrt(np.mean(moe_part ** 2))), near


SMALL = [
    # dtype, H, E, K, I, Is, seq_lens, padded_len, residual scale
    (wk.BF16, 512, 8, 2, 256, 192, (700,), None, 0.05),
    (wk.BF16, 256, 16, 4, 320, 128, (300, 129, 7), 300, 0.03),
    (wk.BF16, 512, 64, 8, 128, 256, (600,), None, 0.05),
    (wk.F32, 256, 8, 2, 128, 128, (64,), None, 0.05),
    (wk.F32, 192, 8, 3, 192, 64, (150, 37), 160, 0.05),
]


@pytest.mark.parametrize("dtype,H,E,K,I,Is,seq,plen,hs", SMALL)
def test_forward_norm_residual_small(dtype, H, E, K, I, Is, seq, plen, hs):
    _say(f"[norm] forward_norm_residual dtype={dtype} H={H} E={E} K={K} seq={seq}")
    d, pad = _case(dtype, H, E, K, I, Is, seq, plen, 7, hs)
    sentinel = 0.75 if pad is not None else None
    out, idx, w, cnt = _gpu_forward_nr(upload(d), K, pad, sentinel)
    rel, moe_rms, _ = _check_nr(d, K, pad, out, idx, w, cnt)
    # the residual does not swamp the layer's part in these cases
    hrms = float(np.sqrt(np.nanmean(as_f64(d["x"][(pad == 0) if pad is not None else
                                                   slice(None)]) ** 2)))
    assert moe_rms > 0.2 * hrms
    if pad is not None:
        assert np.all(as_f64(out[pad == 1]) == 0.75)


def test_forward_norm_residual_in_place():
    _say("[norm] forward_norm_residual in place")
    d, pad = _case(wk.BF16, 256, 16, 4, 320, 128, (300, 129, 7), 300, 9, 0.03)
    out, idx, w, cnt = _gpu_forward_nr(upload(d), 4, pad, inplace=True)
    _check_nr(d, 4, pad, out, idx, w, cnt)
    # padding rows keep h (NaN here) untouched
    assert np.array_equal(out[pad == 1], d["x"][pad == 1])


def test_forward_norm_residual_multichunk():
    """157 token blocks: the router kernel splits H = 512 into 3 slices of
    3, 3 and 2 chunks, so its load pipeline runs whole periods and both tail
    lengths while it writes the normalised rows (every chunk of a real row
    exactly once); padding rows hold NaN and keep the sentinel."""
    _say("[norm] forward_norm_residual multi-chunk slices T=20000 H=512")
    d, pad = _case(wk.BF16, 512, 64, 8, 128, 128, (19667,), 20000, 11, 0.05)
    out, idx, w, cnt = _gpu_forward_nr(upload(d), 8, pad, 0.75)
    real = np.nonzero(pad == 0)[0]
    pick = np.random.default_rng(3).choice(real, 40, replace=False)
    rows = np.unique(np.concatenate([real[:4], real[-4:], pick]))
    _check_nr(d, 8, pad, out, idx, w, cnt, rows=rows)
    assert np.all(as_f64(out[pad == 1]) == 0.75)


def test_forward_norm_residual_full_size():
    _say("[norm] forward_norm_residual full size image_1024")
    wl = wk.workload("image_1024", 0)
    d = wk.make_inputs(wl, 0)
    d["norm_w"] = wk.make_norm_weight(wl.shape, 0)
    pad = d["pad_mask"] if wl.T != wl.T_valid else None
    out, idx, w, cnt = _gpu_forward_nr(upload(d), wl.shape.K, pad)
    rows = np.random.default_rng(0).choice(wl.T, 48, replace=False)
    _check_nr(d, wl.shape.K, pad, out, idx, w, cnt, rows=np.sort(rows))


@pytest.mark.parametrize("H,T,pad_rows", [(512, 700, 0), (256, 333, 40), (4096, 4131, 0),
                                           (512, 20000, 333)])
def test_fused_norm_routes_match_plain_forward_on_rmsnorm(H, T, pad_rows):
    """The block forward normalises inside its router kernel (bf16): its
    normalised rows must be hi3_moe_rmsnorm's bit for bit, so its routes and
    counts equal those of hi3_moe_forward on hi3_moe_rmsnorm(h), bit for bit
    (the router weights' fp32 bits included)."""
    import moe_decoder_ffn_amd as m
    _say(f"[norm] fused norm routes H={H} T={T} pad_rows={pad_rows}")
    E, K = 64, 8
    shape = wk.LayerShape(H=H, E=E, K=K, I=128, Is=128, dtype=wk.BF16)
    wl = wk.custom(shape, (T - pad_rows,), T)
    d = wk.make_inputs(wl, 17)
    d["w_router"] = d["w_router"] * np.float32(3.0)
    d["norm_w"] = wk.make_norm_weight(shape, 17)
    pad = d["pad_mask"] if pad_rows else None
    dd = upload(d)
    padd = to_dev(pad) if pad is not None else None
    _, idx_b, w_b, cnt_b = m.moe_forward_norm_residual(
        dd["x"], dd["norm_w"], dd["w_router"], dd["w13"], dd["w2"], dd["ws13"], dd["ws2"], K,
        pad_mask=padd, return_routes=True)
    xn = torch.zeros_like(dd["x"])
    m.hi3_moe_rmsnorm(dd["x"], dd["norm_w"], 1e-5, padd, xn)
    _, idx_p, w_p, cnt_p = m.moe_forward(xn, dd["w_router"], dd["w13"], dd["w2"], dd["ws13"],
                                         dd["ws2"], K, pad_mask=padd, return_routes=True)
    torch.cuda.synchronize()
    assert torch.equal(idx_b, idx_p) and torch.equal(cnt_b, cnt_p)
    assert torch.equal(w_b.view(torch.int32), w_p.view(torch.int32))
