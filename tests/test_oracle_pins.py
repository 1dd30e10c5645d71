"""Pins of the CPU oracle against facts that do not come from the oracle:
worked examples with hand-derived closed forms, library routines (numpy
float64 matmul / softmax / stable argsort / bincount), special cases that
reduce to a dense MLP or to a full softmax mixture, brute force, and
invariants. Each is chosen so a plausible mistake (dropped term, swapped
up/gate halves, wrong expert offset, wrong tie rule, wrong renormalisation,
padding leaks) fails at least one of them."""
import json
import math
import os

import numpy as np
import pytest

import oracle
import workloads as wk

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _small(dtype, T=24, H=128, E=8, K=2, I=64, Is=64, seed=3, seq_lens=None, skew=False):
    shape = wk.LayerShape(H=H, E=E, K=K, I=I, Is=Is, dtype=dtype)
    wl = wk.custom(shape, seq_lens or (T,), skew=skew)
    return wl, wk.make_inputs(wl, seed)


def _as_f64(a):
    if a.dtype == np.uint16:
        return wk.bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def _round_like(v, dtype):
    """Round fp64 values to the layer dtype (bf16 via the oracle's own
    direct rounding, itself pinned in test_bf16_rounding below)."""
    if dtype == wk.BF16:
        return wk.bf16_bits_to_f32(oracle.round_bf16(v)).astype(np.float64)
    return v.astype(np.float32).astype(np.float64)


# ---------------------------------------------------------------- rounding

def test_bf16_rounding():
    # Values exactly representable in fp32: direct rounding equals the
    # generator's fp32 -> bf16 round-to-nearest-even.
    rng = np.random.default_rng(0)
    v = rng.standard_normal(20000).astype(np.float32)
    v = np.concatenate([v, v * 1e-30, v * 1e30]).astype(np.float32)
    got = oracle.round_bf16(v.astype(np.float64))
    assert np.array_equal(got, wk.f32_to_bf16_bits(v))
    # Ties go to even; a value just above a tie rounds up even when fp32
    # would have rounded it onto the tie first (one rounding, not two).
    cases = {
        1.0 + 2.0 ** -8: 1.0,                       # tie -> even (1.0)
        1.0 + 3 * 2.0 ** -8: 1.0 + 2.0 ** -6,       # tie -> even
        1.0 + 2.0 ** -8 + 2.0 ** -40: 1.0 + 2.0 ** -7,
        -(1.0 + 2.0 ** -8 + 2.0 ** -40): -(1.0 + 2.0 ** -7),
        1.7615941559557646: 1.7578125,
    }
    got = wk.bf16_bits_to_f32(oracle.round_bf16(np.array(list(cases)))).astype(np.float64)
    assert np.array_equal(got, np.array(list(cases.values())))


# ---------------------------------------------------------------- router

@pytest.mark.parametrize("E", [4, 8])
@pytest.mark.parametrize("dtype", [wk.F32, wk.BF16])
def test_topk_tie_worked_example(E, dtype):
    g = _load("topk_tie.json")
    H = 64
    rng = np.random.default_rng(1)
    wr = rng.standard_normal((E, H)).astype(np.float32)
    wr[:, 0] = 0.0
    wr[:4, 0] = g["inputs"]["router_column_0"]
    if E > 4:
        wr[4:, :] = 0.0
    x = np.zeros((1, H), np.float32)
    x[0, 0] = 1.0
    if dtype == wk.BF16:
        x = wk.f32_to_bf16_bits(x)
    r = oracle.route(x, wr, K=2)
    assert r["idx"][0].tolist() == g["expected"]["idx"]
    # the router runs in fp32: a few fp32 ulps
    np.testing.assert_allclose(r["w"][0], g["expected"]["w"], rtol=4e-7)
    if E == 4:
        np.testing.assert_allclose(r["probs"][0], g["expected"]["probs"], rtol=4e-7)


def test_uniform_router():
    # W_r = 0: every probability is 1/E, the tie rule picks experts 0..K-1
    # and each renormalised weight is exactly 1/K.
    wl, d = _small(wk.BF16, E=8, K=4)
    r = oracle.route(d["x"], np.zeros_like(d["w_router"]), K=4)
    assert np.all(r["probs"] == 1.0 / 8)
    assert np.all(r["idx"] == np.arange(4))
    assert np.all(r["w"] == 0.25)


def test_nan_logits_rank_last():
    # A NaN logit counts as -infinity: a router row of NaN makes that
    # expert's logit NaN for every token; it gets probability 0, is never
    # selected, and the other experts' selection and weights are those of
    # the router without that expert (closed form: the same top-K over the
    # remaining logits, renormalised the same way).
    wl, d = _small(wk.BF16, T=30, E=8, K=3, seed=12)
    wr = d["w_router"] * np.float32(10.0)
    bad = wr.copy()
    bad[2] = np.nan
    r = oracle.route(d["x"], bad, K=3)
    assert np.all(r["idx"] != 2) and np.all(r["probs"][:, 2] == 0.0)
    keep = [e for e in range(8) if e != 2]
    r7 = oracle.route(d["x"], wr[keep], K=3)
    assert np.array_equal(r["idx"], np.array(keep)[r7["idx"]])
    np.testing.assert_allclose(r["w"], r7["w"], rtol=1e-6)
    # a row whose input is NaN: every logit is NaN, all count as -infinity,
    # and the tie rule takes experts 0..K-1
    x = d["x"].copy()
    x[5] = wk.BF16_NAN
    r = oracle.route(x, wr, K=3)
    assert np.array_equal(r["idx"][5], [0, 1, 2])


def test_selection_survives_fp32_underflow():
    # One expert's logit is far above the rest, so every other fp32
    # probability underflows to 0 (or a subnormal) and many tie in p. The
    # selection must still be the exact order of the probabilities, i.e. of
    # the logits: the second pick is the second-largest logit.
    E, H = 16, 64
    rng = np.random.default_rng(3)
    wr = rng.standard_normal((E, H)).astype(np.float32) * np.float32(0.1)
    wr[:, 0] = 0.0
    wr[11, 0] = 200.0
    x = rng.standard_normal((4, H)).astype(np.float32)
    x[:, 0] = 1.0
    r = oracle.route(x, wr, K=3)
    l64 = x.astype(np.float64) @ wr.astype(np.float64).T
    for t in range(4):
        order = np.argsort(-l64[t], kind="stable")[:3]
        assert r["idx"][t].tolist() == order.tolist()
        assert r["w"][t, 0] == 1.0 and np.all(r["w"][t, 1:] < 1e-30)


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("E,K", [(8, 2), (16, 5), (64, 8)])
def test_route_invariants_and_library(seed, E, K):
    wl, d = _small(wk.BF16, T=64, H=256, E=E, K=K, seed=seed)
    # Wider router weights than the N(0, 0.02) default so probabilities
    # spread out and the selection is not trivially near-uniform.
    wr = d["w_router"] * np.float32(10.0)
    r = oracle.route(d["x"], wr, K=K)
    idx, w, probs, logits = r["idx"], r["w"], r["probs"], r["logits"]
    # weights: sum to 1 (fp32: within 2K units of 2^-24), non-increasing,
    # ids distinct and in range
    np.testing.assert_allclose(w.astype(np.float64).sum(1), 1.0, rtol=0, atol=2 * K * 2.0 ** -24)
    assert np.all(np.diff(w, axis=1) <= 0)
    assert np.all((idx >= 0) & (idx < E))
    assert all(len(set(row)) == K for row in idx.tolist())
    # logits: numpy float64 matmul, rounded to fp32 (at most 1 ulp apart,
    # the C loop and BLAS sum in different orders)
    ref_logits = (_as_f64(d["x"]) @ wr.astype(np.float64).T).astype(np.float32)
    ulp = np.spacing(np.abs(ref_logits))
    assert np.all(np.abs(logits - ref_logits) <= ulp)
    # softmax over all experts: numpy float64 on the oracle's fp32 logits
    # (the oracle evaluates it in fp32: a few ulps, relative)
    l64 = logits.astype(np.float64)
    ref_p = np.exp(l64 - l64.max(1, keepdims=True))
    ref_p /= ref_p.sum(1, keepdims=True)
    np.testing.assert_allclose(probs, ref_p, rtol=2e-6, atol=1e-37)
    # top-k: stable argsort of the negated logits (lower index first on
    # ties), and the same order as float64 probabilities
    ref_idx = np.argsort(-logits, axis=1, kind="stable")[:, :K]
    assert np.array_equal(idx, ref_idx)
    assert np.array_equal(idx, np.argsort(-ref_p, axis=1, kind="stable")[:, :K])
    # renormalisation identity: renorm(topK(softmax(l))) = softmax(l[idx])
    sel = np.take_along_axis(l64, idx.astype(np.int64), 1)
    ref_w = np.exp(sel - sel.max(1, keepdims=True))
    ref_w /= ref_w.sum(1, keepdims=True)
    np.testing.assert_allclose(w, ref_w, rtol=2e-6, atol=1e-37)


# ---------------------------------------------------------------- expert

@pytest.mark.parametrize("dtype", [wk.F32, wk.BF16])
def test_swiglu_up_first_worked_example(dtype):
    g = _load("swiglu_up_first.json")
    E, K, H, I = 8, 2, 64, 64
    wl, d = _small(dtype, T=1, H=H, E=E, K=K, I=I, Is=I)
    one = np.float32(1.0)
    z = lambda a: np.zeros_like(a)
    w13, w2 = z(d["w13"]), z(d["w2"])
    if dtype == wk.BF16:
        c = lambda v: wk.f32_to_bf16_bits(np.float32(v))
    else:
        c = lambda v: np.float32(v)
    w13[:, 0, 0] = c(1.0)       # up row 0
    w13[:, I, 0] = c(2.0)       # gate row 0
    w2[:, 0, 0] = c(1.0)
    x = np.zeros((1, H), np.float32)
    x[0, 0] = one
    if dtype == wk.BF16:
        x = wk.f32_to_bf16_bits(x)
    r = oracle.moe(x, d["w_router"], w13, w2, z(d["ws13"]), z(d["ws2"]), K=K)
    out = _as_f64(r["out"])[0]
    want = g["expected"]["out0_bf16" if dtype == wk.BF16 else "out0_f32"]
    if dtype == wk.BF16:
        # exact: h is rounded to bf16, far from a rounding boundary
        assert out[0] == want
    else:
        # the fp32 gate weights sum to 1 within an ulp
        np.testing.assert_allclose(out[0], want, rtol=2.5e-7)
    assert abs(out[0] - g["expected"]["swapped_layout_value"]) > 0.1
    assert np.all(out[1:] == 0)
    np.testing.assert_allclose(r["exact"][0, 0], want, rtol=2.5e-7)


def _numpy_swiglu(x64, w13, w2, dtype):
    """Dense SwiGLU MLP on many rows with numpy float64 matmuls; h rounded
    to the layer dtype like any stored activation."""
    I = w13.shape[0] // 2
    uv = x64 @ _as_f64(w13).T
    u, g = uv[:, :I], uv[:, I:]
    h = _round_like(g / (1.0 + np.exp(-g)) * u, dtype)
    return h @ _as_f64(w2).T


@pytest.mark.parametrize("dtype", [wk.F32, wk.BF16])
def test_single_expert_reduces_to_two_mlps(dtype):
    # E = 1, K = 1: the gate weight is 1 and the layer is
    # SwiGLU_0(x) + SwiGLU_shared(x), two dense MLPs.
    wl, d = _small(dtype, T=16, H=128, E=1, K=1, I=64, Is=96)
    r = oracle.moe(d["x"], d["w_router"], d["w13"], d["w2"], d["ws13"], d["ws2"], K=1)
    assert np.all(r["idx"] == 0) and np.all(r["w"] == 1.0)
    x64 = _as_f64(d["x"])
    ref = _numpy_swiglu(x64, d["w13"][0], d["w2"][0], dtype) + \
        _numpy_swiglu(x64, d["ws13"], d["ws2"], dtype)
    scale = np.sqrt(np.mean(ref ** 2))
    # h may round differently where BLAS and the C loop disagree in the last
    # fp64 bit right at a rounding boundary: allow a few such flips.
    assert np.max(np.abs(r["exact"] - ref)) <= 1e-3 * scale
    assert np.mean(np.abs(r["exact"] - ref) > 1e-12 * scale) < 0.01


@pytest.mark.parametrize("dtype", [wk.F32, wk.BF16])
def test_k_equals_e_is_full_softmax_mixture(dtype):
    # K = E: renormalisation is the identity, so the layer is the full
    # softmax mixture sum_e p_e * Expert_e(x) + Shared(x).
    E = 8
    wl, d = _small(dtype, T=12, H=128, E=E, K=E, I=64, Is=64, seed=5)
    wr = d["w_router"] * np.float32(20.0)
    r = oracle.moe(d["x"], wr, d["w13"], d["w2"], d["ws13"], d["ws2"], K=E)
    x64 = _as_f64(d["x"])
    logits = (x64 @ wr.astype(np.float64).T).astype(np.float32).astype(np.float64)
    p = np.exp(logits - logits.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    ref = _numpy_swiglu(x64, d["ws13"], d["ws2"], dtype)
    for e in range(E):
        ref += p[:, e:e + 1] * _numpy_swiglu(x64, d["w13"][e], d["w2"][e], dtype)
    scale = np.sqrt(np.mean(ref ** 2))
    # gate weights are fp32 (router precision): ~1e-7 relative differences
    assert np.max(np.abs(r["exact"] - ref)) <= 1e-5 * scale
    # and the gate weights are the probabilities, in descending order
    ref_w = -np.sort(-p, axis=1)
    np.testing.assert_allclose(r["w"], ref_w, rtol=2e-6)


@pytest.mark.parametrize("dtype", [wk.F32, wk.BF16])
@pytest.mark.parametrize("E,K", [(8, 2), (8, 3), (16, 4)])
def test_sparse_dispatch_equals_dense_bruteforce(dtype, E, K):
    wl, d = _small(dtype, T=20, H=128, E=E, K=K, I=64, Is=64, seed=7)
    wr = d["w_router"] * np.float32(10.0)
    r = oracle.moe(d["x"], wr, d["w13"], d["w2"], d["ws13"], d["ws2"], K=K)
    dense = oracle.moe_dense(d["x"], d["w13"], d["w2"], d["ws13"], d["ws2"],
                             r["idx"], r["w"])
    scale = np.sqrt(np.mean(dense ** 2))
    assert np.max(np.abs(r["exact"] - dense)) <= 1e-12 * scale


def test_routes_in_replace_router():
    wl, d = _small(wk.BF16, T=10, E=8, K=2, seed=9)
    args = (d["x"], d["w_router"], d["w13"], d["w2"], d["ws13"], d["ws2"])
    r = oracle.moe(*args, K=2)
    r2 = oracle.moe(*args, K=2, idx=r["idx"], w=r["w"])
    assert np.array_equal(r["out"], r2["out"])
    other = (r["idx"] + 1) % 8
    r3 = oracle.moe(*args, K=2, idx=other, w=r["w"])
    dense = oracle.moe_dense(d["x"], d["w13"], d["w2"], d["ws13"], d["ws2"], other, r["w"])
    assert np.max(np.abs(r3["exact"] - dense)) <= 1e-12 * np.sqrt(np.mean(dense ** 2))
    assert not np.array_equal(r3["out"], r["out"])


# ---------------------------------------------------------------- padding

@pytest.mark.parametrize("dtype", [wk.F32, wk.BF16])
def test_padding_rows_untouched_and_not_read(dtype):
    wl, d = _small(dtype, H=128, E=8, K=2, I=64, Is=64, seq_lens=(5, 9, 3), seed=11)
    pad = d["pad_mask"]
    assert pad.sum() > 0
    x = d["x"]
    # padding rows hold NaN (set by the generator): reading any would show
    assert np.all(np.isnan(_as_f64(x)[pad.astype(bool)]))
    sentinel = np.full((wl.T, 128), 0x1234 if dtype == wk.BF16 else 7.25, x.dtype)
    args = (x, d["w_router"], d["w13"], d["w2"], d["ws13"], d["ws2"])
    r = oracle.moe(*args, K=2, pad_mask=pad, out=sentinel.copy())
    assert np.array_equal(r["out"][pad == 1], sentinel[pad == 1])
    assert not np.any(np.isnan(_as_f64(r["out"][pad == 0])))
    assert np.all(r["idx"][pad == 1] == -1) and np.all(r["w"][pad == 1] == 0)
    # real rows equal a run on the compacted real rows, bit for bit
    keep = pad == 0
    r2 = oracle.moe(x[keep], d["w_router"], d["w13"], d["w2"], d["ws13"], d["ws2"], K=2)
    assert np.array_equal(r["out"][keep], r2["out"])
    rr = oracle.route(x, d["w_router"], K=2, pad_mask=pad)
    assert np.all(rr["idx"][pad == 1] == -1)


def test_row_subset_and_determinism():
    wl, d = _small(wk.BF16, T=30, E=8, K=2, seed=13)
    args = (d["x"], d["w_router"], d["w13"], d["w2"], d["ws13"], d["ws2"])
    a = oracle.moe(*args, K=2)
    b = oracle.moe(*args, K=2)
    assert np.array_equal(a["out"], b["out"]) and np.array_equal(a["exact"], b["exact"])
    rows = np.array([29, 3, 17, 3])
    c = oracle.moe(*args, K=2, rows=rows)
    assert np.array_equal(c["out"], a["out"][rows])


def test_bf16_tolerance_attainable():
    # The final bf16 rounding alone must stay inside the 2e-2 * RMS bar,
    # otherwise no implementation could meet it.
    wl, d = _small(wk.BF16, T=64, H=512, E=8, K=2, I=256, Is=256, seed=17)
    r = oracle.moe(d["x"], d["w_router"], d["w13"], d["w2"], d["ws13"], d["ws2"], K=2)
    rounded = wk.bf16_bits_to_f32(r["out"]).astype(np.float64)
    rms = np.sqrt(np.mean(r["exact"] ** 2))
    assert np.max(np.abs(rounded - r["exact"])) <= 0.0127 * 1.2 * rms


# ---------------------------------------------------------------- dispatch

def test_dispatch_definition_bruteforce():
    rng = np.random.default_rng(0)
    T, K, E = 37, 3, 6
    idx = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    idx[[4, 20]] = -1     # padding rows
    d = oracle.dispatch(idx, E)
    # brute force: walk experts in order, tokens in order, k in order
    slots = []
    for e in range(E):
        for t in range(T):
            for k in range(K):
                if idx[t, k] == e:
                    slots.append((t, k))
    assert d["perm_token"].tolist() == [t for t, _ in slots]
    for s, (t, k) in enumerate(slots):
        assert d["slot_of"][t, k] == s
    assert np.all(d["slot_of"][[4, 20]] == -1)
    assert d["counts"].tolist() == [sum(1 for t, k in slots if idx[t, k] == e) for e in range(E)]
    assert d["offsets"][0] == 0 and d["offsets"][-1] == len(slots)
    assert np.array_equal(np.diff(d["offsets"]), d["counts"])
