"""GPU parity of the whole layer (hi3_moe_forward) against the CPU oracle:
small cases compared on every row (several GEMM tiles, ragged tails,
padding, edge cases), the full-size workloads on every row's routes and on
sampled rows' outputs, plus determinism."""
import json
import os
import sys

import numpy as np
import pytest

import oracle
import workloads as wk

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

from parity import (as_f64, check_output, check_routes, oracle_rows, to_dev,  # noqa: E402
                    to_host, upload)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def gpu_forward(dd, K, pad=None, sentinel=None, side_stream=None):
    """Runs hi3_moe_forward (hi3_moe_forward_overlap with a side stream) on
    device inputs dd; returns host out, idx, w, counts."""
    import moe_decoder_ffn_amd as m
    x = dd["x"]
    T, H = x.shape
    E = dd["w_router"].shape[0]
    if sentinel is None:
        out = torch.zeros_like(x)
    else:
        out = torch.full_like(x, sentinel)
    padd = to_dev(pad) if pad is not None else None
    out, idx, w, cnt = m.moe_forward(x, dd["w_router"], dd["w13"], dd["w2"], dd["ws13"],
                                     dd["ws2"], K, pad_mask=padd, out=out, return_routes=True,
                                     side_stream=side_stream)
    torch.cuda.synchronize()
    return to_host(out), to_host(idx), to_host(w), to_host(cnt)


def full_check(d, K, pad=None, sentinel=None, rows=None):
    """Forward on the GPU, then: routes of all rows; counts; outputs of
    `rows` (all real rows by default) against the oracle."""
    E = d["w_router"].shape[0]
    dtype = wk.BF16 if d["x"].dtype == np.uint16 else wk.F32
    out, idx, w, cnt = gpu_forward(upload(d), K, pad, sentinel)
    ref = oracle.route(d["x"], d["w_router"], K, pad_mask=pad)
    near, ref_idx, ref_w = check_routes(idx, w, ref, pad, E, K)
    assert np.array_equal(cnt, np.bincount(idx[idx >= 0], minlength=E))
    valid = np.ones(len(idx), bool) if pad is None else pad == 0
    if rows is None:
        rows = np.nonzero(valid)[0]
    exact = oracle_rows(d, K, rows, ref_idx, ref_w, pad)
    rel = check_output(out[rows], exact, dtype)
    return out, idx, w, cnt, near, rel


SMALL = [
    # name, dtype, H, E, K, I, Is, seq_lens, padded_len
    ("tiny_f32", wk.F32, 256, 8, 2, 128, 128, (64,), None),
    ("f32_ragged", wk.F32, 192, 8, 3, 192, 64, (150, 37), 160),
    ("bf16_tiles", wk.BF16, 512, 8, 2, 256, 192, (700,), None),
    ("bf16_e16_pad", wk.BF16, 256, 16, 4, 320, 128, (300, 129, 7), 300),
    ("bf16_e64_k8", wk.BF16, 512, 64, 8, 128, 256, (600,), None),
    ("bf16_one_token", wk.BF16, 256, 8, 2, 128, 128, (1,), None),
]


@pytest.mark.parametrize("name,dtype,H,E,K,I,Is,seq,plen", SMALL)
def test_forward_small_all_rows(name, dtype, H, E, K, I, Is, seq, plen):
    _say(f"[forward] {name}")
    shape = wk.LayerShape(H=H, E=E, K=K, I=I, Is=Is, dtype=dtype)
    wl = wk.custom(shape, seq, plen)
    d = wk.make_inputs(wl, 7)
    d["w_router"] = d["w_router"] * np.float32(5.0)
    pad = d["pad_mask"] if wl.T != wl.T_valid else None
    sentinel = 0.75 if pad is not None else None
    out, idx, *_ = full_check(d, K, pad, sentinel)
    if pad is not None:
        # padding rows keep the sentinel (never written), nothing is NaN
        assert np.all(as_f64(out[pad == 1]) == 0.75)
        assert np.isfinite(as_f64(out[pad == 0])).all()


@pytest.mark.parametrize("H,I,Is", [(64, 64, 64), (128, 64, 128), (64, 128, 192), (192, 320, 64)])
def test_forward_short_reductions(H, I, Is):
    """Reductions of 1 to 5 k steps of 64 on the default (256-row) tiles:
    the weight ring runs its copies two steps ahead and repeats the last
    step near the end, so the first and last steps meet at these sizes."""
    _say(f"[forward] short reductions H={H} I={I} Is={Is}")
    shape = wk.LayerShape(H=H, E=2, K=1, I=I, Is=Is, dtype=wk.BF16)
    d = wk.make_inputs(wk.custom(shape, (600,)), 13)
    full_check(d, 1, None, None)


@pytest.mark.parametrize("T", [1, 64, 65, 112, 113, 128, 129, 192, 193, 256, 257, 513])
def test_forward_tile_boundaries(T):
    """One expert (E = K = 1), so every row goes to it and the row-tile
    edges are hit by construction. Up to 112 rows per expert the layer runs
    the streaming tiles (64 rows). Above, both projections use 256-row tiles
    with a half-height body at <= 128 rows and a three-quarter body at
    <= 192."""
    _say(f"[forward] tile boundaries T={T}")
    shape = wk.LayerShape(H=256, E=1, K=1, I=128, Is=192, dtype=wk.BF16)
    d = wk.make_inputs(wk.custom(shape, (T,)), 11)
    out, idx, w, cnt, *_ = full_check(d, 1)
    assert np.all(idx == 0) and np.all(w == 1.0) and cnt[0] == T


def test_forward_nan_rows_keep_dispatch_in_bounds():
    # Real rows whose input is NaN and a NaN router row: routing still picks
    # exactly K experts per row (a NaN logit counts as -infinity), so the
    # dispatch sizes hold; the NaN rows give NaN outputs and every other row
    # matches the oracle.
    _say("[forward] NaN rows and a NaN router row")
    shape = wk.LayerShape(H=256, E=16, K=4, I=128, Is=128, dtype=wk.BF16)
    d = wk.make_inputs(wk.custom(shape, (200,)), 5)
    d["x"][[3, 111]] = wk.BF16_NAN
    d["w_router"] = d["w_router"] * np.float32(5.0)
    d["w_router"][9] = np.nan
    out, idx, w, cnt = gpu_forward(upload(d), 4)
    assert int(cnt.sum()) == 200 * 4 and cnt[9] == 0
    ok = np.setdiff1d(np.arange(200), [3, 111])
    ref = oracle.route(d["x"], d["w_router"], 4)
    near, ref_idx, ref_w = check_routes(idx[ok], w[ok], {k: v[ok] for k, v in ref.items()},
                                        None, 16, 4)
    exact = oracle.moe(d["x"], d["w_router"], d["w13"], d["w2"], d["ws13"], d["ws2"], K=4,
                       rows=ok, idx=ref_idx, w=ref_w)["exact"]
    check_output(out[ok], exact, wk.BF16)


@pytest.mark.parametrize("dtype", [wk.F32, wk.BF16])
def test_forward_k_equals_e(dtype):
    _say(f"[forward] K=E dtype={dtype}")
    shape = wk.LayerShape(H=256, E=8, K=8, I=128, Is=128, dtype=dtype)
    d = wk.make_inputs(wk.custom(shape, (64,)), 3)
    d["w_router"] = d["w_router"] * np.float32(20.0)
    full_check(d, 8)


@pytest.mark.parametrize("dtype", [wk.F32, wk.BF16])
def test_forward_swiglu_up_first_worked_example(dtype):
    g = json.load(open(os.path.join(GOLDEN, "swiglu_up_first.json")))
    E, K, H, I = 8, 2, 256, 128
    shape = wk.LayerShape(H=H, E=E, K=K, I=I, Is=I, dtype=dtype)
    d = wk.make_inputs(wk.custom(shape, (5,)), 0)
    c = (lambda v: wk.f32_to_bf16_bits(np.float32(v))) if dtype == wk.BF16 else np.float32
    for k in ("w13", "w2", "ws13", "ws2"):
        d[k][...] = 0
    d["w13"][:, 0, 0] = c(1.0)
    d["w13"][:, I, 0] = c(2.0)
    d["w2"][:, 0, 0] = c(1.0)
    x = np.zeros((5, H), np.float32)
    x[:, 0] = 1.0
    d["x"] = wk.f32_to_bf16_bits(x) if dtype == wk.BF16 else x
    out, *_ = gpu_forward(upload(d), K)
    out = as_f64(out)
    want = g["expected"]["out0_bf16" if dtype == wk.BF16 else "out0_f32"]
    if dtype == wk.BF16:
        assert np.all(out[:, 0] == want), out[:, 0]
    else:
        # fp32: device expf and the fp32 gate weights, a few ulps
        np.testing.assert_allclose(out[:, 0], want, rtol=5e-7)
    assert np.all(np.abs(out[:, 0] - g["expected"]["swapped_layout_value"]) > 0.1)
    assert np.all(out[:, 1:] == 0)


def test_forward_edge_cases():
    import moe_decoder_ffn_amd as m
    shape = wk.LayerShape(H=256, E=16, K=2, I=128, Is=128, dtype=wk.BF16)
    # all rows padding: nothing written, counts zero
    _say("[forward] all padding")
    d = wk.make_inputs(wk.custom(shape, (0, 0), padded_len=40), 0)
    out, idx, w, cnt = gpu_forward(upload(d), 2, d["pad_mask"], sentinel=3.0)
    assert np.all(as_f64(out) == 3.0) and np.all(idx == -1) and np.all(cnt == 0)
    # an empty expert and a one-row expert: router rows that never / once win
    _say("[forward] empty + one-row experts")
    d = wk.make_inputs(wk.custom(shape, (300,)), 1)
    wr = d["w_router"] * np.float32(3.0)
    wr[5] = 0.0
    wr[5, 0] = -100.0        # expert 5 loses everywhere x[:,0] > 0 ...
    xf = wk.bf16_bits_to_f32(d["x"]).copy()
    xf[:, 0] = np.abs(xf[:, 0]) + 0.5
    xf[17, 0] = -3.0         # ... except token 17, where it wins
    d["x"] = wk.f32_to_bf16_bits(xf)
    d["w_router"] = wr
    out, idx, w, cnt, *_ = full_check(d, 2)
    assert cnt[5] == 1 and 5 in idx[17]
    wr2 = wr.copy()
    wr2[5, 0] = -1000.0
    xf[17, 0] = 1.0
    d["x"] = wk.f32_to_bf16_bits(xf)
    d["w_router"] = wr2
    out, idx, w, cnt, *_ = full_check(d, 2)
    assert cnt[5] == 0


def test_forward_deterministic():
    shape = wk.LayerShape(H=512, E=64, K=8, I=256, Is=256, dtype=wk.BF16)
    d = upload(wk.make_inputs(wk.custom(shape, (999,)), 5))
    a = gpu_forward(d, 8)
    b = gpu_forward(d, 8)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


def _hip_events(n):
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    evs = []
    for _ in range(n):
        e = ctypes.c_void_p()
        assert hip.hipEventCreate(ctypes.byref(e)) == 0
        evs.append(e.value)
    return hip, evs


@pytest.mark.parametrize("T,E,K,Is,H", [(700, 8, 2, 192, 512), (999, 64, 8, 320, 512),
                                        (4131, 64, 8, 256, 512), (1000, 8, 2, 192, 320),
                                        (100, 8, 2, 192, 512), (512, 64, 8, 256, 512)])
def test_forward_overlap_same_bits(T, E, K, Is, H):
    """hi3_moe_forward_overlap runs the shared expert's GEMMs on the caller's
    side stream (dense launches over rows 0 .. T-1); hi3_moe_forward keeps
    them in the grouped list on one stream. Every output element is the
    same reduction in the same order either way (k steps of 64, the same
    MFMA and epilogue), so every output bit, route and count must match,
    and so must the instrumented forward with and without the side stream.
    H = 320 leaves the down projections a partial column tile and 5 k
    steps; T = 100 and 512 (at most 112 rows per expert) run the routed
    GEMMs on the streaming tiles while the dense launches keep 256-row
    tiles."""
    import moe_decoder_ffn_amd as m
    _say(f"[forward] overlap vs one stream T={T} E={E} K={K} Is={Is} H={H}")
    shape = wk.LayerShape(H=H, E=E, K=K, I=256, Is=Is, dtype=wk.BF16)
    assert m.hi3_moe_forward_shared_on_side(T, shape.H, E, K, shape.I, Is, wk.BF16, False)
    assert not m.hi3_moe_forward_shared_on_side(T, shape.H, E, K, shape.I, Is, wk.BF16, True)
    assert not m.hi3_moe_forward_shared_on_side(T, shape.H, E, K, shape.I, Is, wk.F32, False)
    d = upload(wk.make_inputs(wk.custom(shape, (T,)), 11))
    one = gpu_forward(d, K)
    side_stream = torch.cuda.Stream()
    side = gpu_forward(d, K, side_stream=side_stream)
    for u, v in zip(side, one):
        assert np.array_equal(u, v)
    # the same stream given as the side stream: one stream
    same = gpu_forward(d, K, side_stream=torch.cuda.current_stream())
    for u, v in zip(same, one):
        assert np.array_equal(u, v)
    x = d["x"]
    ws = m.workspace_for(x, E, K, shape.I, Is)
    for sst in (None, side_stream):
        out = torch.zeros_like(x)
        idx = torch.empty((T, K), dtype=torch.int32, device="cuda")
        w = torch.empty((T, K), dtype=torch.float32, device="cuda")
        cnt = torch.empty((E,), dtype=torch.int32, device="cuda")
        hip, evs = _hip_events(m.HI3_NUM_STAGES + 1)
        try:
            m.hi3_moe_forward_instrumented(x, d["w_router"], d["w13"], d["w2"], d["ws13"],
                                           d["ws2"], None, K, out, idx, w, cnt, ws, evs,
                                           torch.cuda.current_stream(), sst)
            torch.cuda.synchronize()
        finally:
            for e in evs:
                hip.hipEventDestroy(e)
        for u, v in zip(one, (out, idx, w, cnt)):
            assert np.array_equal(u, to_host(v))


def test_forward_concurrent_host_threads():
    """Two host threads, each with a main and a side stream of its own,
    enqueue overlapped and plain forwards at the same time (the library
    keeps no state between calls): every result matches a single-threaded
    forward bit for bit."""
    import threading
    import moe_decoder_ffn_amd as m
    _say("[forward] two host threads")
    shape = wk.LayerShape(H=512, E=64, K=8, I=256, Is=320, dtype=wk.BF16)
    cases = ((999, 21), (1500, 22))
    inputs = [upload(wk.make_inputs(wk.custom(shape, (T,)), seed)) for T, seed in cases]
    ref = [gpu_forward(d, shape.K) for d in inputs]
    results = [None, None]
    errors = []

    def run(i):
        try:
            st, side = torch.cuda.Stream(), torch.cuda.Stream()
            d = inputs[i]
            with torch.cuda.stream(st):
                outs = [m.moe_forward(d["x"], d["w_router"], d["w13"], d["w2"], d["ws13"],
                                      d["ws2"], shape.K, return_routes=True,
                                      side_stream=side if j % 2 == 0 else None)
                        for j in range(4)]
            st.synchronize()
            results[i] = [[to_host(t) for t in o] for o in outs]
        except Exception as e:  # reported by the main thread
            errors.append(e)

    threads = [threading.Thread(target=run, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not errors, errors
    for i in range(2):
        assert results[i] is not None
        for o in results[i]:
            for u, v in zip(ref[i], o):
                assert np.array_equal(u, v)


def test_forward_overlap_graph_capture():
    """An overlapped forward captured into a graph (the side stream joins
    the capture through the call's fork and leaves it at the join) while
    another host thread runs eager forwards on streams of its own: every
    replay, with eager work and synchronisations between replays, matches
    the eager result bit for bit, and so does every eager forward of the
    other thread. The forward's kernels write every workspace byte they read
    (no memset in the graph)."""
    import threading
    import moe_decoder_ffn_amd as m
    _say("[forward] graph capture of the overlapped forward")
    shape = wk.LayerShape(H=512, E=64, K=8, I=256, Is=320, dtype=wk.BF16)
    T = 999
    d = upload(wk.make_inputs(wk.custom(shape, (T,)), 31))
    d2 = upload(wk.make_inputs(wk.custom(shape, (T,)), 32))
    ref = gpu_forward(d, shape.K)
    ref2 = gpu_forward(d2, shape.K)
    x = d["x"]
    ws = m.workspace_for(x, shape.E, shape.K, shape.I, shape.Is)
    out = torch.zeros_like(x)
    idx = torch.empty((T, shape.K), dtype=torch.int32, device="cuda")
    w = torch.empty((T, shape.K), dtype=torch.float32, device="cuda")
    cnt = torch.empty((shape.E,), dtype=torch.int32, device="cuda")
    side = torch.cuda.Stream()
    args = (x, d["w_router"], d["w13"], d["w2"], d["ws13"], d["ws2"], None, shape.K, out, idx,
            w, cnt, ws)
    # warm up on a side stream of torch's choosing, as graph capture wants
    warm = torch.cuda.Stream()
    warm.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(warm):
        m.hi3_moe_forward_overlap(*args, side_stream=side)
    torch.cuda.current_stream().wait_stream(warm)
    torch.cuda.synchronize()
    stop = threading.Event()
    errors, eager = [], []
    # the other thread's streams and buffers exist before the capture starts,
    # so nothing is created or allocated while it runs
    st2, side2 = torch.cuda.Stream(), torch.cuda.Stream()
    ws2 = m.workspace_for(d2["x"], shape.E, shape.K, shape.I, shape.Is)
    bufs2 = (torch.zeros_like(d2["x"]), torch.empty((T, shape.K), dtype=torch.int32, device="cuda"),
             torch.empty((T, shape.K), dtype=torch.float32, device="cuda"),
             torch.empty((shape.E,), dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()

    def other():
        try:
            with torch.cuda.stream(st2):
                while not stop.is_set() and len(eager) < 20:
                    m.hi3_moe_forward_overlap(d2["x"], d2["w_router"], d2["w13"], d2["w2"],
                                              d2["ws13"], d2["ws2"], None, shape.K, *bufs2, ws2,
                                              side_stream=side2, stream=st2)
                    st2.synchronize()
                    eager.append([to_host(t) for t in bufs2])
        except Exception as e:
            errors.append(e)

    th = threading.Thread(target=other)
    th.start()
    try:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, capture_error_mode="thread_local"):
            m.hi3_moe_forward_overlap(*args, side_stream=side)
        for rep in range(3):
            out.zero_()
            idx.fill_(-7)
            g.replay()
            torch.cuda.synchronize()
            for u, v in zip(ref, (out, idx, w, cnt)):
                assert np.array_equal(u, to_host(v)), f"replay {rep}"
            # eager work between replays
            gpu_forward(d2, shape.K)
    finally:
        stop.set()
        th.join(timeout=120)
    assert not errors, errors
    assert eager
    for o in eager:
        for u, v in zip(ref2, o):
            assert np.array_equal(u, v)


# ---------------------------------------------------------------- full size

@pytest.fixture(scope="module")
def full_weights():
    _say("[forward] generating full-size expert weights")
    w = wk.make_expert_weights(wk.FULL, 0)
    dev = upload(w)
    return w, dev


def _sample_rows(valid_rows, n, seed):
    rng = np.random.default_rng(seed)
    pick = rng.choice(valid_rows, size=min(n, valid_rows.size), replace=False)
    return np.unique(np.concatenate([valid_rows[:2], valid_rows[-2:], pick]))


# Workloads whose every real row's output is compared with the oracle (the
# 1024x1024 image sequence: about 40 s of oracle time on 16 host cores); the
# others compare every row's routes and a sample of rows' outputs.
ALL_ROWS = ("image_1024",)


@pytest.mark.parametrize("name", ["image_1024", "batch8_512", "skew_16k", "padded_mixed",
                                  "image_512", "prompt_512"])
def test_forward_full_size(full_weights, name):
    """The full-size workloads through hi3_moe_forward_overlap, the entry
    point the benchmark times (its side stream is used where every row is
    real): routes of every row, counts, and outputs against the oracle."""
    w_host, w_dev = full_weights
    wl = wk.workload(name, 0)
    sh = wl.shape
    _say(f"[forward] full size {name}: T={wl.T}, real {wl.T_valid}")
    x, pad = wk.make_x(wl, 0)
    wr = wk.make_router_weight(sh, 0, skew=wl.skew)
    padarg = pad if wl.T != wl.T_valid else None
    dd = dict(w_dev)
    dd["x"] = to_dev(x)
    dd["w_router"] = to_dev(wr)
    out, idx, w, cnt = gpu_forward(dd, sh.K, padarg, sentinel=0.5 if padarg is not None else None,
                                   side_stream=torch.cuda.Stream())
    del dd
    ref = oracle.route(x, wr, sh.K, pad_mask=padarg)
    near, ref_idx, ref_w = check_routes(idx, w, ref, padarg, sh.E, sh.K)
    assert np.array_equal(cnt, np.bincount(idx[idx >= 0], minlength=sh.E))
    valid_rows = np.nonzero(pad == 0)[0]
    if name in ALL_ROWS:
        rows = valid_rows
    else:
        rows = _sample_rows(valid_rows, 24, 1)
        rows = np.unique(np.concatenate([rows, np.nonzero(near)[0][:4]]))
    _say(f"  oracle on {rows.size} rows")
    d = dict(w_host)
    d["x"] = x
    d["w_router"] = wr
    exact = oracle_rows(d, sh.K, rows, ref_idx, ref_w, padarg)
    stats = {}
    check_output(out[rows], exact, sh.dtype, name, stats)
    rec = {"workload": name, "rows_compared": int(rows.size), "real_rows": int(valid_rows.size),
           "near_tie_rows": int(near.sum()), "near_tie_rows_compared": int(near[rows].sum()),
           **{k: (round(v, 5) if isinstance(v, float) else v) for k, v in stats.items()},
           "load_max_over_mean": round(float(cnt.max() / cnt.mean()), 3),
           "load_min": int(cnt.min())}
    _say("  parity " + json.dumps(rec))
    if padarg is not None:
        assert np.all(as_f64(out[pad == 1]) == 0.5)
    if wl.skew:
        assert cnt[:4].min() > 3.0 * cnt.mean() and cnt[-4:].max() < 0.05 * cnt.mean()
