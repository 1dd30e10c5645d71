"""GPU parity of the router (hi3_moe_route) against the CPU oracle."""
import json
import os
import sys

import numpy as np
import pytest

import oracle
import workloads as wk

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from parity import as_f64, check_routes, to_dev, to_host  # noqa: E402

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def run_route(x, wr, K, pad=None, counts=True):
    import moe_decoder_ffn_amd as m
    xd, wd = to_dev(x), to_dev(wr)
    T = x.shape[0]
    E = wr.shape[0]
    pd = to_dev(pad) if pad is not None else None
    idx = torch.full((T, K), -7, dtype=torch.int32, device="cuda")
    w = torch.full((T, K), -7.0, dtype=torch.float32, device="cuda")
    cnt = torch.full((E,), -7, dtype=torch.int32, device="cuda") if counts else None
    ws = m.workspace_for(xd, E, K)
    m.hi3_moe_route(xd, wd, pd, K, idx, w, cnt, ws)
    torch.cuda.synchronize()
    return to_host(idx), to_host(w), (to_host(cnt) if counts else None)


CASES = [
    # name, dtype, T, H, E, K, seq_lens(None = no padding), router scale
    ("tiny_f32", wk.F32, 64, 256, 8, 2, None, 1.0),
    ("f32_wide", wk.F32, 333, 512, 64, 8, None, 5.0),
    ("bf16_e64", wk.BF16, 1000, 512, 64, 8, None, 1.0),
    ("bf16_e40_pad", wk.BF16, 0, 1024, 40, 6, (300, 17, 255), 3.0),
    ("bf16_e8_k8", wk.BF16, 257, 256, 8, 8, None, 10.0),
    ("bf16_e33_k1", wk.BF16, 95, 320, 33, 1, None, 10.0),
    # 157 token blocks: 3 slices of the 8 chunks (3, 3, 2), so the logit
    # kernel runs whole periods of its load pipeline and both tail lengths
    ("bf16_multichunk", wk.BF16, 20000, 512, 64, 8, None, 1.0),
]


@pytest.mark.parametrize("name,dtype,T,H,E,K,seq,scale", CASES)
def test_route_parity(name, dtype, T, H, E, K, seq, scale):
    _say(f"[route] {name}")
    shape = wk.LayerShape(H=H, E=E, K=K, I=64, Is=64, dtype=dtype)
    wl = wk.custom(shape, seq or (T,))
    x, pad = wk.make_x(wl, 1)
    wr = wk.make_router_weight(shape, 1) * np.float32(scale)
    padarg = pad if seq else None
    idx, w, cnt = run_route(x, wr, K, padarg)
    ref = oracle.route(x, wr, K, pad_mask=padarg)
    check_routes(idx, w, ref, padarg, E, K)
    valid = idx[idx >= 0]
    assert np.array_equal(cnt, np.bincount(valid, minlength=E))


def test_route_full_size_image_1024():
    wl = wk.workload("image_1024")
    _say(f"[route] full size T={wl.T}")
    x, pad = wk.make_x(wl, 0)
    wr = wk.make_router_weight(wl.shape, 0)
    idx, w, cnt = run_route(x, wr, wl.shape.K)
    ref = oracle.route(x, wr, wl.shape.K)
    near, _, _ = check_routes(idx, w, ref, None, wl.shape.E, wl.shape.K)
    _say(f"  near-tie rows: {int(near.sum())}")
    assert np.array_equal(cnt, np.bincount(idx.reshape(-1), minlength=wl.shape.E))


def test_route_tie_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "topk_tie.json")))
    for dtype in (wk.F32, wk.BF16):
        H, E = 64, 8
        wr = np.zeros((E, H), np.float32)
        wr[:4, 0] = g["inputs"]["router_column_0"]
        wr[:4, 1:] = np.random.default_rng(0).standard_normal((4, H - 1)).astype(np.float32)
        x = np.zeros((3, H), np.float32)
        x[:, 0] = 1.0
        if dtype == wk.BF16:
            x = wk.f32_to_bf16_bits(x)
        idx, w, _ = run_route(x, wr, 2)
        assert idx.tolist() == [g["expected"]["idx"]] * 3
        np.testing.assert_allclose(w, [g["expected"]["w"]] * 3, rtol=0, atol=1e-6)


def test_route_uniform_router():
    # W_r = 0: all probabilities equal, experts 0..K-1 in order, weights 1/K.
    shape = wk.LayerShape(H=256, E=64, K=8, I=64, Is=64, dtype=wk.BF16)
    x, _ = wk.make_x(wk.custom(shape, (100,)), 0)
    idx, w, cnt = run_route(x, np.zeros((64, 256), np.float32), 8)
    assert np.all(idx == np.arange(8)) and np.all(w == np.float32(0.125))
    assert cnt.tolist() == [100] * 8 + [0] * 56


def test_route_all_padding():
    shape = wk.LayerShape(H=256, E=16, K=4, I=64, Is=64, dtype=wk.BF16)
    x, _ = wk.make_x(wk.custom(shape, (70,)), 0)
    pad = np.ones(70, np.uint8)
    idx, w, cnt = run_route(x, wk.make_router_weight(shape, 0), 4, pad)
    assert np.all(idx == -1) and np.all(w == 0) and np.all(cnt == 0)


def test_route_nan_logits_select_exactly_k():
    # A NaN router row (that expert's logit is NaN for every token) and real
    # rows whose input is NaN (every logit NaN): a NaN logit counts as
    # -infinity, so every real row still selects exactly K distinct experts
    # and the counts total T * K; ids match the oracle on every row.
    _say("[route] NaN logits")
    shape = wk.LayerShape(H=512, E=64, K=8, I=64, Is=64, dtype=wk.BF16)
    x, _ = wk.make_x(wk.custom(shape, (300,)), 4)
    x[[7, 150]] = wk.BF16_NAN
    wr = wk.make_router_weight(shape, 4)
    wr[5] = np.nan
    idx, w, cnt = run_route(x, wr, 8)
    ref = oracle.route(x, wr, 8)
    # expert 5 is chosen only by the two all-NaN rows, which tie every expert
    # at -infinity and take experts 0..7
    assert int(cnt.sum()) == 300 * 8 and cnt[5] == 2
    assert np.all(np.sort(idx, 1)[:, 1:] != np.sort(idx, 1)[:, :-1])
    assert np.array_equal(idx[[7, 150]], ref["idx"][[7, 150]])
    ok = np.setdiff1d(np.arange(300), [7, 150])
    check_routes(idx[ok], w[ok], {k: v[ok] for k, v in ref.items()}, None, 64, 8)
