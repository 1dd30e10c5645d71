"""The seeded input generator: sizes of the named workloads, determinism,
independence from the thread count, padding layout, and the skewed-router
load construction (checked with the oracle's router)."""
import numpy as np
import pytest

import oracle
import workloads as wk


def test_named_workload_sizes():
    assert wk.workload("tiny_f32").T == 64
    # 32 prompt + 1 timestep + 64*64 image + 2 suffix tokens
    assert wk.workload("image_1024").T == 4131
    assert wk.workload("batch8_512").T == 8 * 1123 == 8984
    assert wk.workload("skew_16k").T == 16384
    for seed in (0, 1, 2):
        wl = wk.workload("padded_mixed", seed)
        lens = wl.seq_lens
        assert len(lens) == 4
        imgs = [48 * 80, 64 * 64, 80 * 48, 32 * 128]
        for n, im in zip(lens, imgs):
            assert 64 <= n - im <= 200
        assert wl.T == 4 * max(lens)
        assert wl.T_valid == sum(lens)
        m = wl.pad_mask().reshape(4, -1)
        for b, n in enumerate(lens):
            assert m[b, :n].sum() == 0 and m[b, n:].all()


def test_flop_per_token():
    assert wk.flop_per_valid_token(wk.FULL) == 680_001_536


def test_determinism_and_thread_independence(monkeypatch):
    shape = wk.LayerShape(H=128, E=8, K=2, I=64, Is=64, dtype=wk.BF16)
    wl = wk.custom(shape, (700, 300), padded_len=700)
    a = wk.make_inputs(wl, 5)
    monkeypatch.setattr(wk, "_X_ROWS_PER_CHUNK", wk._X_ROWS_PER_CHUNK)
    monkeypatch.setattr(wk, "_threads", lambda: 1)
    b = wk.make_inputs(wl, 5)
    for k in a:
        assert np.array_equal(a[k], b[k], equal_nan=True), k
    c = wk.make_inputs(wl, 6)
    assert not np.array_equal(a["w13"], c["w13"])


def test_distributions_and_padding():
    shape = wk.LayerShape(H=256, E=8, K=2, I=128, Is=128, dtype=wk.BF16)
    wl = wk.custom(shape, (900, 400), padded_len=900)
    d = wk.make_inputs(wl, 0)
    x = wk.bf16_bits_to_f32(d["x"])
    pad = d["pad_mask"].astype(bool)
    assert np.all(np.isnan(x[pad])) and not np.any(np.isnan(x[~pad]))
    assert abs(x[~pad].std() - 1.0) < 0.01 and abs(x[~pad].mean()) < 0.01
    for k in ("w13", "w2", "ws13", "ws2"):
        v = wk.bf16_bits_to_f32(d[k])
        assert abs(v.std() - 0.02) < 0.0005, k
    assert d["w_router"].dtype == np.float32 and abs(d["w_router"].std() - 0.02) < 0.001


def test_bf16_conversion_ties_to_even():
    v = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -1.0 - 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -23],
                 np.float32)
    got = wk.bf16_bits_to_f32(wk.f32_to_bf16_bits(v))
    assert got.tolist() == [1.0, 1.0 + 2.0 ** -6, -1.0, 1.0 + 2.0 ** -7]
    assert wk.f32_to_bf16_bits(np.array([np.nan], np.float32))[0] == 0x7FC0


def test_skewed_router_load():
    # Router weights of the skew workload at full width, routed by the
    # oracle on a sample of 2048 tokens: experts 0..3 get about 4x the mean
    # load, the last four almost none.
    wl = wk.workload("skew_16k")
    sh = wl.shape
    w = wk.make_weights(wk.LayerShape(sh.H, sh.E, sh.K, 64, 64, sh.dtype), 0, skew=True)
    x, _ = wk.make_x(wk.custom(sh, (2048,)), 0)
    r = oracle.route(x, w["w_router"], K=sh.K)
    load = np.bincount(r["idx"].reshape(-1), minlength=sh.E) / (2048 * sh.K / sh.E)
    assert np.all(load[:4] > 3.0), load[:4]
    assert np.all(load[-4:] < 0.05), load[-4:]
    assert np.all(load[4:-4] < 1.5)
