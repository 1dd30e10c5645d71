"""GPU test of hi3_moe_forward_noalloc, the forward for callers that cannot
allocate: called through the C ABI and compared with hi3_moe_forward (the
same kernels on a workspace of the caller's) bit for bit, on two calls in a
row, the second with a smaller input, so that the scratch's leftovers from
the first call cannot change the second's result."""
import sys

import numpy as np
import pytest

import workloads as wk

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

from parity import to_dev, to_host  # noqa: E402


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _both(m, x, wr, w13, w2, ws13, ws2, pad, K):
    """(hi3_moe_forward result, hi3_moe_forward_noalloc result), host arrays
    of out, idx, w, counts; and the free device memory around the no-alloc
    call."""
    T = x.shape[0]
    E = wr.shape[0]
    res = []
    free = None
    for noalloc in (False, True):
        out = torch.full_like(x, 0.25)
        idx = torch.full((T, K), -9, dtype=torch.int32, device="cuda")
        w = torch.full((T, K), 7.0, dtype=torch.float32, device="cuda")
        cnt = torch.full((E,), -9, dtype=torch.int32, device="cuda")
        if noalloc:
            torch.cuda.synchronize()
            before = torch.cuda.mem_get_info()[0]
            m.hi3_moe_forward_noalloc(x, wr, w13, w2, ws13, ws2, pad, K, out, idx, w, cnt)
            torch.cuda.synchronize()
            free = (before, torch.cuda.mem_get_info()[0])
        else:
            ws = m.workspace_for(x, E, K, w13.shape[1] // 2, ws13.shape[0] // 2)
            m.hi3_moe_forward(x, wr, w13, w2, ws13, ws2, pad, K, out, idx, w, cnt, ws)
            torch.cuda.synchronize()
            del ws
        res.append([to_host(t) for t in (out, idx, w, cnt)])
    return res[0], res[1], free


def _check(ref, got):
    for name, u, v in zip(("out", "idx", "w", "counts"), ref, got):
        assert u.shape == v.shape and np.array_equal(u, v), name


def test_noalloc_matches_forward_small_shape():
    import moe_decoder_ffn_amd as m
    shape = wk.LayerShape(H=512, E=64, K=8, I=256, Is=320, dtype=wk.BF16)
    for T, seed, padded in ((3000, 1, None), (999, 2, 1100)):
        _say(f"[noalloc] small shape T={T} padded={padded}")
        wl = wk.custom(shape, (T,), padded)
        d = wk.make_inputs(wl, seed)
        pad = d["pad_mask"] if wl.T != wl.T_valid else None
        dd = {k: to_dev(v) for k, v in d.items() if k != "pad_mask"}
        ref, got, free = _both(m, dd["x"], dd["w_router"], dd["w13"], dd["w2"], dd["ws13"],
                               dd["ws2"], to_dev(pad) if pad is not None else None, shape.K)
        _check(ref, got)
        if pad is not None:
            assert np.all(wk.bf16_bits_to_f32(got[0][pad == 1]) == 0.25)


def test_noalloc_full_shape_two_calls():
    import moe_decoder_ffn_amd as m
    sh = wk.FULL
    w = {k: to_dev(v) for k, v in wk.make_expert_weights(sh, 0).items()}
    wr = to_dev(wk.make_router_weight(sh, 0))
    frees = []
    # the second call is smaller and padded
    for seq, padded in (((600,), None), ((100, 37), 100)):
        wl = wk.custom(sh, seq, padded)
        _say(f"[noalloc] full shape T={wl.T} real {wl.T_valid}")
        x, pad = wk.make_x(wl, 3)
        padd = to_dev(pad) if wl.T != wl.T_valid else None
        ref, got, free = _both(m, to_dev(x), wr, w["w13"], w["w2"], w["ws13"], w["ws2"], padd,
                               sh.K)
        _check(ref, got)
        frees.append(free)
    # after the first call on this device, a call allocates no device memory
    assert frees[1][0] == frees[1][1], frees


def test_noalloc_rejects_sizes_beyond_scratch():
    import moe_decoder_ffn_amd as m
    sh = wk.FULL
    T = 700  # needs more than HI3_NOALLOC_SCRATCH_BYTES at this shape
    assert m.hi3_moe_workspace_size(T, sh.H, sh.E, sh.K, sh.I, sh.Is, wk.BF16) > \
        m.HI3_NOALLOC_SCRATCH_BYTES
    p = 1 << 20
    st = m.lib.hi3_moe_forward_noalloc(p, p, p, p, p, p, None, T, sh.H, sh.E, sh.K, sh.I, sh.Is,
                                       wk.BF16, p, None, None, None, None)
    assert st == m.HI3_E_SCRATCH
