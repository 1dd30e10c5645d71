"""Helpers for the GPU parity tests: upload of generated inputs, and the
comparison rules against the CPU oracle.

Rules (all against the oracle on the same seeded inputs):

* Routes. For a real row let gap = l_(K) - l_(K+1) of the oracle's fp32
  logits sorted descending. Where gap > 1e-4 the GPU's K expert ids must be
  exactly the oracle's (as sets), and its weights must match the oracle's
  per expert within ROUTE_W_TOL. Where gap <= 1e-4 both selections are
  correct: the GPU ids must be K distinct ids whose weights match the
  oracle's probabilities at those ids, renormalised; the row's output is then
  compared with the oracle run on the GPU's ids. Every row's ids are ordered
  by non-increasing weight, equal weights by ascending id. Padding rows:
  ids -1, weights 0.
* Outputs. max |gpu - oracle| over the compared real rows must be at most
  2e-2 * RMS(oracle output) for bf16 layers and 1e-5 * RMS for fp32 layers,
  against the oracle's fp64 value before the final rounding. For bf16 this
  literal bar applies wherever the oracle's own correctly rounded output
  meets it (max |bf16(exact) - exact| <= 2e-2 RMS over the compared rows);
  only where even that misses the bar (an output element so far above the
  RMS that half a bf16 ulp exceeds 2e-2 RMS) may an element instead be
  within one bf16 ulp of the exact value.
* Integer work (counts, offsets, permutations, gathered rows) is compared
  bit for bit.

ROUTE_W_TOL: the GPU's fp32 logits differ from the oracle's by a few 1e-6 at
full size (fp32 accumulation over H = 4096 terms whose absolute sum is about
50); a renormalised weight w moves by at most about 2 w dl, well below
2e-5.
"""
import numpy as np
import torch

import oracle
import workloads as wk

GAP_TOL = 1e-4
ROUTE_W_TOL = 2e-5
OUT_TOL = {wk.BF16: 2e-2, wk.F32: 1e-5}
# per-term relative bound of the bf16 gradients (check_grad)
GRAD_REL = 3 * 2.0 ** -8


def to_dev(a, device="cuda"):
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def to_host(t):
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def as_f64(a):
    if a.dtype == np.uint16:
        return wk.bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def upload(d):
    return {k: to_dev(v) for k, v in d.items()}


def check_routes(gpu_idx, gpu_w, ref, pad, E, K):
    """Returns (near_rows, ref_idx_for_rows, ref_w_for_rows): the routes the
    oracle should use per row (its own where the gap is clear, the GPU's
    where it is not)."""
    T = gpu_idx.shape[0]
    valid = np.ones(T, bool) if pad is None else pad == 0
    assert np.all(gpu_idx[~valid] == -1) and np.all(gpu_w[~valid] == 0)
    logits = ref["logits"]
    if K < E:
        srt = -np.sort(-logits, axis=1)
        gap = srt[:, K - 1].astype(np.float64) - srt[:, K].astype(np.float64)
    else:
        gap = np.full(T, np.inf)
    near = valid & (gap <= GAP_TOL)
    firm = valid & ~near
    gi = gpu_idx.astype(np.int64)
    # ids in range and distinct, order by non-increasing weight
    v = gi[valid]
    assert v.size == 0 or (v.min() >= 0 and v.max() < E)
    assert np.all(np.sort(v, 1)[:, 1:] != np.sort(v, 1)[:, :-1]) if K > 1 else True
    gw = gpu_w[valid].astype(np.float64)
    assert np.all(np.diff(gw, axis=1) <= 0)
    # firm rows: same sets, weights per id
    bad = np.nonzero(firm & np.any(np.sort(gi, 1) != np.sort(ref["idx"], 1), axis=1))[0]
    assert bad.size == 0, f"route mismatch at rows {bad[:10]} (gaps {gap[bad[:10]]})"
    rows = np.nonzero(firm)[0]
    dense_g = np.zeros((rows.size, E))
    dense_r = np.zeros((rows.size, E))
    np.put_along_axis(dense_g, gi[rows], gpu_w[rows].astype(np.float64), 1)
    np.put_along_axis(dense_r, ref["idx"][rows].astype(np.int64), ref["w"][rows], 1)
    err = np.abs(dense_g - dense_r).max() if rows.size else 0.0
    assert err <= ROUTE_W_TOL, f"route weight error {err}"
    # near rows: weights = oracle probabilities at the GPU's ids, renormalised
    ref_idx = ref["idx"].copy()
    ref_w = ref["w"].copy()
    for t in np.nonzero(near)[0]:
        p = ref["probs"][t, gi[t]]
        w = p / p.sum()
        assert np.abs(w - gpu_w[t]).max() <= ROUTE_W_TOL
        ref_idx[t] = gi[t]
        ref_w[t] = w
    return near, ref_idx, ref_w


def bf16_ulp(v):
    """Spacing of bf16 numbers at |v| (8 significant bits)."""
    a = np.abs(v)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def check_output(gpu_rows, exact_rows, dtype, what="", stats=None):
    """Asserts the output rule above; returns max |err| / RMS. stats (a
    dict), when given, receives the rule applied and the measured ratios."""
    g = as_f64(gpu_rows)
    rms = float(np.sqrt(np.mean(exact_rows ** 2))) if exact_rows.size else 0.0
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    if g.size == 0:
        return 0.0
    diff = np.abs(g - exact_rows)
    err = float(diff.max())
    if dtype == wk.F32:
        tol = OUT_TOL[dtype] * rms
        rule = "1e-5 * RMS"
        assert err <= tol, f"{what}: max err {err:.4g} > {tol:.4g} (1e-5 * RMS {rms:.4g})"
    else:
        # how far the oracle's own output moves when rounded once to bf16
        rounding = float(np.max(np.abs(as_f64(oracle.round_bf16(exact_rows)) - exact_rows)))
        if rounding <= OUT_TOL[dtype] * rms:
            rule = "literal: max err <= 2e-2 * RMS"
            assert err <= OUT_TOL[dtype] * rms, (
                f"{what}: max err / RMS {err / rms:.4f} > 2e-2 (the rounded oracle output "
                f"itself is within {rounding / rms:.4f} * RMS)")
        else:
            rule = "max(2e-2 * RMS, 1 ulp): the rounded oracle output misses 2e-2 * RMS"
            bound = np.maximum(OUT_TOL[dtype] * rms, bf16_ulp(exact_rows))
            bad = np.argwhere(diff > bound)
            assert bad.size == 0, (f"{what}: {len(bad)} elements outside max(2e-2 * RMS, 1 ulp); "
                                   f"first {bad[:3].tolist()}, max err / RMS {err / rms:.4f}")
        erms = float(np.sqrt(np.mean(diff ** 2)))
        assert erms <= 5e-3 * rms, f"{what}: RMS error {erms / rms:.4g} * RMS"
        if stats is not None:
            stats["oracle_rounding_over_rms"] = rounding / rms
            stats["rms_err_over_rms"] = erms / rms
    if stats is not None:
        stats.update(rule=rule, max_err_over_rms=err / rms, rms=rms, elements=int(g.size))
    return err / rms


def check_grad(gpu, exact, mag, dtype, what=""):
    """Gradient rule (the backward's outputs): fp32 layers as the forward
    (max |err| <= 1e-5 RMS). bf16 layers, every element:
        |err| <= ulp(exact) + GRAD_REL * mag,  GRAD_REL = 3 * 2^-8
    where mag is the sum of the absolute values of the terms the oracle sums
    into that element. Each term differs from the oracle's by at most three
    bf16 roundings of relative size <= 2^-8 (bf16's unit roundoff, 8
    significant bits): at most two on the GPU's path (an MFMA operand and
    its producer), and, for terms holding the SwiGLU activation h, the
    oracle's own rounding of h from the exact pre-activation, which may fall
    on the other side of a rounding midpoint than the GPU's rounding from
    its fp32 pre-activation (the two h then differ by one ulp); fp32 sums add
    far less. The result is rounded once more (<= 1 ulp of the exact value,
    allowing for a binade change). Plus, for the whole tensor, RMS error <=
    5e-3 RMS: the roundings are unbiased, so a systematic mistake (a missing
    or doubled row) shows there even where the per-element worst case is
    wide. Differences below 2^-16 of the tensor's largest magnitude are not
    resolved: the oracle's router values are fp32, and its evaluation of the
    softmax chain leaves residues of that order where the exact derivative is
    zero (the logits of unselected experts).
    Returns max |err| / RMS."""
    g = as_f64(gpu)
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    if g.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(exact ** 2)))
    diff = np.abs(g - exact)
    err = float(diff.max())
    if dtype == wk.F32:
        tol = OUT_TOL[dtype] * rms
        assert err <= tol, f"{what}: max err {err:.4g} > {tol:.4g} (1e-5 * RMS {rms:.4g})"
    else:
        bound = bf16_ulp(exact) + GRAD_REL * mag + 2.0 ** -16 * float(np.max(mag))
        bad = np.argwhere(diff > bound)
        assert bad.size == 0, (f"{what}: {len(bad)} elements outside ulp + 3 * 2^-8 * sum|terms|; "
                               f"first {bad[:3].tolist()}, worst err / bound "
                               f"{float((diff / bound).max()):.3f}")
        erms = float(np.sqrt(np.mean(diff ** 2)))
        assert erms <= 5e-3 * rms, f"{what}: RMS error {erms / rms:.4g} * RMS"
    return err / max(rms, 1e-300)


def check_grad_chunked(gpu, exact, mag, dtype, what=""):
    """check_grad for a large gradient, one slice of the first axis at a
    time (the same per-element bound; the RMS error rule over the whole
    tensor from accumulated sums), so that no full-size float64 temporary
    is made. Returns max |err| / RMS."""
    assert dtype == wk.BF16
    mmax = float(np.max(mag))
    sq_err = sq_ref = 0.0
    worst = 0.0
    n = 0
    for i in range(exact.shape[0]):
        g = as_f64(gpu[i])
        e = exact[i]
        assert np.isfinite(g).all(), f"{what}[{i}]: non-finite output"
        diff = np.abs(g - e)
        bound = bf16_ulp(e) + GRAD_REL * mag[i] + 2.0 ** -16 * mmax
        bad = np.argwhere(diff > bound)
        assert bad.size == 0, (f"{what}[{i}]: {len(bad)} elements outside ulp + 3 * 2^-8 * "
                               f"sum|terms|; first {bad[:3].tolist()}, worst err / bound "
                               f"{float((diff / bound).max()):.3f}")
        sq_err += float(np.sum(diff ** 2))
        sq_ref += float(np.sum(e ** 2))
        worst = max(worst, float(diff.max()))
        n += e.size
    rms = np.sqrt(sq_ref / n)
    erms = np.sqrt(sq_err / n)
    assert erms <= 5e-3 * rms, f"{what}: RMS error {erms / rms:.4g} * RMS"
    return worst / max(rms, 1e-300)


def oracle_rows(d, K, rows, idx, w, pad=None):
    """The oracle's layer output at `rows` using the given routes for them."""
    r = oracle.moe(d["x"], d["w_router"], d["w13"], d["w2"], d["ws13"], d["ws2"], K=K,
                   pad_mask=pad, rows=rows, idx=idx[rows], w=w[rows])
    return r["exact"]
