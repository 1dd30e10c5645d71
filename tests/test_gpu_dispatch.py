"""GPU dispatch (hi3_moe_dispatch) against the oracle's definition of the
expert grouping (bincount + stable argsort); integer work, compared bit for
bit, gathered rows byte for byte."""
import sys

import numpy as np
import pytest

import oracle
import workloads as wk

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

from parity import to_dev, to_host  # noqa: E402


def _routes(T, E, K, seed, skew=False):
    rng = np.random.default_rng(seed)
    if skew:
        p = np.ones(E)
        p[:4] = 40.0
        p[-3:] = 0.0
        p /= p.sum()
        idx = np.stack([rng.choice(E, K, replace=False, p=p) for _ in range(T)])
    else:
        idx = np.stack([rng.permutation(E)[:K] for _ in range(T)])
    return idx.astype(np.int32)


@pytest.mark.parametrize("T,H,E,K,dtype,npad,skew", [
    (64, 256, 8, 2, wk.F32, 0, False),
    (1000, 512, 64, 8, wk.BF16, 0, False),
    (777, 256, 64, 8, wk.BF16, 123, True),
    (4131, 4096, 64, 8, wk.BF16, 0, False),
    (100, 128, 5, 5, wk.BF16, 7, False),
    (33, 64, 64, 1, wk.F32, 1, False),
])
def test_dispatch_bitwise(T, H, E, K, dtype, npad, skew):
    import moe_decoder_ffn_amd as m
    print(f"[dispatch] T={T} E={E} K={K} pad={npad}", file=sys.stderr, flush=True)
    shape = wk.LayerShape(H=H, E=E, K=K, I=64, Is=64, dtype=dtype)
    x, _ = wk.make_x(wk.custom(shape, (T,)), 2)
    idx = _routes(T, E, K, 3, skew)
    pad = np.zeros(T, np.uint8)
    pad[np.random.default_rng(4).choice(T, npad, replace=False)] = 1
    idx_in = idx.copy()
    idx_in[pad == 1] = 12345  # ids of padding rows must not be read
    xd = to_dev(x)
    off = torch.full((E + 1,), -9, dtype=torch.int32, device="cuda")
    perm = torch.full((T * K,), -9, dtype=torch.int32, device="cuda")
    slot = torch.full((T * K,), -9, dtype=torch.int32, device="cuda")
    xs = torch.zeros((T * K, H), dtype=xd.dtype, device="cuda")
    ws = m.workspace_for(xd, E, K)
    m.hi3_moe_dispatch(to_dev(idx_in), to_dev(pad), xd, E, off, perm, slot, xs, ws)
    torch.cuda.synchronize()
    ref_idx = idx.copy()
    ref_idx[pad == 1] = -1
    ref = oracle.dispatch(ref_idx, E)
    S = int(ref["offsets"][-1])
    assert S == (T - npad) * K
    assert np.array_equal(to_host(off), ref["offsets"])
    p = to_host(perm)
    assert np.array_equal(p[:S], ref["perm_token"])
    assert np.all(p[S:] == -9)  # unwritten past S
    assert np.array_equal(to_host(slot).reshape(T, K), ref["slot_of"])
    xs_h = to_host(xs)
    assert np.array_equal(xs_h[:S].view(np.uint8), x[ref["perm_token"]].view(np.uint8))
    assert not np.any(xs_h[S:].view(np.uint8))
