#!/usr/bin/env python3
"""Benchmark of the routed-expert MoE feed-forward layer on one MI355X.

One step = one hi3_moe_forward call over one batch of synthetic tokens, on
one stream: the router, dispatch, grouped [up; gate] + SwiGLU GEMM, grouped
down GEMM (the shared expert's rows ride in both grouped launches) and
combine. Inputs are resident in HBM before timing starts.

Prints one JSON line: tokens/s over the real tokens (the metric), with the
layer's TFLOP/s and fraction of the bf16 MFMA peak, the roofline entry of the
dominant kernel (its duration measured with HIP events recorded on the
launch stream inside the timed region, where it has the GPU to itself),
per-stage times, the same call with the shared expert on a second stream of
the caller's (hi3_moe_forward_overlap) for comparison, the achievable peaks
measured on this GPU next to the published ones, the batch's per-expert
load, and the CPU oracle timed on a bounded sample of the same workload on
this host's cores.
"""
import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as wk  # noqa: E402

METRIC = "MoE-layer tokens/s + TFLOP/s (% bf16 MFMA peak), 64e top-8, H=4096, 1 GPU"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class HipEvents:
    """Raw hipEvent_t handles through the HIP runtime torch already loaded."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                 ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            out.append(e.value)
        return out

    def elapsed_ms(self, a, b):
        self.hip.hipEventSynchronize(b)
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(e)


def stage_bytes(wl):
    """Algorithmic HBM bytes per call of the memory-bound stages."""
    sh = wl.shape
    es = 2 if sh.dtype == wk.BF16 else 4
    Tv, T, H, E, K = wl.T_valid, wl.T, sh.H, sh.E, sh.K
    return {
        # x read once, the fp32 router weight, routes written
        "router": Tv * H * es + E * H * 4 + T * K * 8,
        # K fp32 expert rows + the fp32 shared row read, one output row written
        "combine": Tv * (K * H * 4 + H * 4 + H * es + K * 8),
    }


# Rows per expert below which the grouped GEMMs are bound by reading their
# weights rather than by MFMA: the bf16 ridge, 2.5 PFLOP/s / 8 TB/s = 312
# FLOP per byte, is reached at about 312 rows per expert (each weight byte
# is used for 2 FLOP per row, two bytes per weight).
RIDGE_ROWS = 312


def upgate_bytes(wl, shared=True):
    """Algorithmic HBM bytes of the [up; gate] GEMM: every expert's and (with
    shared) the shared expert's [up; gate] weights once, each routed or
    shared row of x once per use, h written once."""
    sh = wl.shape
    es = 2 if sh.dtype == wk.BF16 else 4
    sf = 1 if shared else 0
    rows = wl.T_valid * (sh.K + sf)
    return (sh.E * 2 * sh.I * sh.H + sf * 2 * sh.Is * sh.H) * es + rows * sh.H * es + \
        (wl.T_valid * sh.K * sh.I + sf * wl.T_valid * sh.Is) * es


def gemm_flops(wl, shared=True):
    """Algorithmic FLOP of the forward's GEMM stages; shared=False when the
    shared expert's GEMMs run on the side stream, outside these stages."""
    sh = wl.shape
    Tv = wl.T_valid
    sf = 1 if shared else 0
    return {
        "gemm_up_gate_swiglu": Tv * (sh.K * 2 * sh.H * 2 * sh.I + sf * 2 * sh.H * 2 * sh.Is),
        "gemm_down": Tv * (sh.K * 2 * sh.I * sh.H + sf * 2 * sh.Is * sh.H),
    }


GEMM_SOURCES = ("moe_decoder_ffn_amd/csrc/gemm.hip", "moe_decoder_ffn_amd/csrc/common.h")


def gemm_source_hash():
    h = hashlib.sha256()
    for rel in GEMM_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload):
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary (FETCH_SIZE + WRITE_SIZE, each scaled by the same counter's
    reading for a plain copy of known size), or None if there is none for
    this workload or the kernel source changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_gemm_up_gate_swiglu_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256") != gemm_source_hash():
        return None
    return int(float(kv["hbm_bytes_per_launch"]))


def copy_calibration(mib):
    """A plain device-to-device copy of known size, for scaling the HBM
    byte counters (run under rocprofv3 --pmc)."""
    import torch
    n = mib * 2 ** 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "launches": 3}), flush=True)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def achievable_peaks(m):
    """What this GPU sustains in practice, beside the published peaks: the
    library's matrix-core probe (bf16 MFMA chains, no memory traffic), a
    dense bf16 GEMM through torch (hipBLASLt), and a device copy through
    torch (bytes read + written per second)."""
    import torch
    hip = HipEvents()
    hip.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    st = torch.cuda.current_stream()
    ev = hip.create(2)

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        hip.hip.hipEventRecord(ev[0], ctypes.c_void_p(st.cuda_stream))
        for _ in range(reps):
            fn()
        hip.hip.hipEventRecord(ev[1], ctypes.c_void_p(st.cuda_stream))
        return hip.elapsed_ms(ev[0], ev[1]) / reps

    g = torch.Generator(device="cuda")
    g.manual_seed(1)
    # operands with the statistics of the layer's (bf16 values of N(0, 1)),
    # whose bit switching sets the clock the matrix cores hold
    bits = torch.randn(8192, device="cuda", generator=g).to(torch.bfloat16)
    out = torch.empty(1024 * 4, dtype=torch.float32, device="cuda")
    flop = [0]

    def probe():
        flop[0] = m.hi3_moe_probe_mfma_bf16(bits, out, 1024, 4096)

    mfma_ms = timed(probe, 3)
    n = 8192
    a = (torch.randn((n, n), device="cuda", generator=g) * 0.02).to(torch.bfloat16)
    b = (torch.randn((n, n), device="cuda", generator=g) * 0.02).to(torch.bfloat16)
    c = torch.empty((n, n), dtype=torch.bfloat16, device="cuda")
    gemm_ms = timed(lambda: torch.mm(a, b, out=c), 5)
    del a, b, c
    nbytes = 1 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    copy_ms = timed(lambda: dst.copy_(src), 5)
    del src, dst
    hip.destroy(ev)
    return {"mfma_bf16_probe_tflops": round(flop[0] / (mfma_ms * 1e-3) / 1e12, 1),
            "hipblaslt_bf16_gemm_8192_tflops": round(2 * n ** 3 / (gemm_ms * 1e-3) / 1e12, 1),
            "device_copy_gbs": round(2 * nbytes / (copy_ms * 1e-3) / 1e9, 1)}


def expert_load(cnt):
    """Per-expert routed rows: how skewed the routing of this batch is."""
    c = np.asarray(cnt, dtype=np.float64)
    mean = c.mean()
    return {"max_over_mean": round(float(c.max() / mean), 3), "min": int(c.min()),
            "max": int(c.max()), "experts_below_1pct_of_mean": int((c < 0.01 * mean).sum())}


def cpu_baseline(wl, d, K, target_s):
    """The CPU oracle as it stands, on a bounded sample of real tokens."""
    import oracle
    pad = d["pad_mask"]
    valid = np.nonzero(pad == 0)[0]
    cores = len(os.sched_getaffinity(0))
    args = (d["x"], d["w_router"], d["w13"], d["w2"], d["ws13"], d["ws2"])
    n = max(1, min(cores, valid.size))
    t0 = time.perf_counter()
    oracle.moe(*args, K=K, pad_mask=pad, rows=valid[:n])
    first = time.perf_counter() - t0
    # grow the sample to about target_s seconds of wall time in total
    n2 = int(min(valid.size - n, max(0, (target_s - first) / max(first, 1e-3) * n)))
    total_n, total_t = n, first
    if n2 > 0:
        t0 = time.perf_counter()
        oracle.moe(*args, K=K, pad_mask=pad, rows=valid[n:n + n2])
        total_t += time.perf_counter() - t0
        total_n += n2
    return {"value": total_n / total_t, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{total_n} real tokens of {wl.name} (full layer per token, fp64 C, "
                      f"OpenMP over tokens), {total_t:.1f} s"}


def norm_residual_bench(args, m, wl, d, dd, pad, ws, stream):
    """Times h + layer(RMSNorm(h)) per step (whole call), against the plain
    layer on already-normalised rows on the same inputs (alternating, one
    stream), and the RMSNorm kernel alone against the HBM roofline (x read,
    normalised rows written): in bf16 the block entry runs no RMSNorm kernel
    (the router kernel normalises), so its cost is the difference."""
    import torch
    sh = wl.shape
    nw = torch.from_numpy(wk.make_norm_weight(sh, args.seed).view(np.int16)).cuda().view(
        torch.bfloat16) if sh.dtype == wk.BF16 else torch.from_numpy(
        wk.make_norm_weight(sh, args.seed)).cuda()
    h = dd["x"]
    out = torch.zeros_like(h)
    xn = torch.empty_like(h)
    m.hi3_moe_rmsnorm(h, nw, 1e-5, pad, xn, stream)
    idx = torch.empty((wl.T, sh.K), dtype=torch.int32, device="cuda")
    wts = torch.empty((wl.T, sh.K), dtype=torch.float32, device="cuda")
    cnt = torch.empty((sh.E,), dtype=torch.int32, device="cuda")
    w = (dd["w_router"], dd["w13"], dd["w2"], dd["ws13"], dd["ws2"])

    def block():
        m.hi3_moe_forward_norm_residual(h, nw, 1e-5, *w, pad, sh.K, out, idx, wts, cnt, ws,
                                        stream)

    def plain():
        m.hi3_moe_forward(xn, *w, pad, sh.K, out, idx, wts, cnt, ws, stream)

    hip = HipEvents()
    hip.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    ev = hip.create(3)
    for _ in range(args.warmup):
        block()
        plain()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        block()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    log(f"[bench] {args.steps} timed steps done")
    blk_ms = pl_ms = 0.0
    for _ in range(args.steps):
        hip.hip.hipEventRecord(ev[0], ctypes.c_void_p(stream.cuda_stream))
        block()
        hip.hip.hipEventRecord(ev[1], ctypes.c_void_p(stream.cuda_stream))
        plain()
        hip.hip.hipEventRecord(ev[2], ctypes.c_void_p(stream.cuda_stream))
        blk_ms += hip.elapsed_ms(ev[0], ev[1])
        pl_ms += hip.elapsed_ms(ev[1], ev[2])
    blk_ms /= args.steps
    pl_ms /= args.steps
    reps = 20
    hip.hip.hipEventRecord(ev[0], ctypes.c_void_p(stream.cuda_stream))
    for _ in range(reps):
        m.hi3_moe_rmsnorm(h, nw, 1e-5, pad, xn, stream)
    hip.hip.hipEventRecord(ev[1], ctypes.c_void_p(stream.cuda_stream))
    norm_ms = hip.elapsed_ms(ev[0], ev[1]) / reps
    hip.destroy(ev)
    es = 2 if sh.dtype == wk.BF16 else 4
    norm_bytes = 2 * wl.T_valid * sh.H * es + sh.H * es
    gbs = norm_bytes / (norm_ms * 1e-3) / 1e9
    tokens_s = wl.T_valid / (ms_per_step * 1e-3)
    line = {
        "metric": METRIC, "value": round(tokens_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if sh.dtype == wk.BF16 else "f32", "data": "synthetic",
        "config": {"workload": wl.name, "entry": "norm_residual", "T": wl.T,
                   "T_valid": wl.T_valid, "H": sh.H, "E": sh.E, "K": sh.K, "I": sh.I,
                   "I_shared": sh.Is, "eps": 1e-5, "seed": args.seed},
        "block_vs_plain": {"block_us": round(blk_ms * 1e3, 1), "plain_us": round(pl_ms * 1e3, 1),
                           "difference_us": round((blk_ms - pl_ms) * 1e3, 1)},
        "stages": {"rmsnorm_kernel_alone": {"us": round(norm_ms * 1e3, 2), "gbs": round(gbs, 1),
                                            "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)}},
        "roofline": None,
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def backward_gemm_flops(wl):
    """Algorithmic FLOP of the backward's GEMM stages (routed + shared)."""
    sh = wl.shape
    Tv = wl.T_valid
    up = Tv * (sh.K * 2 * sh.H * 2 * sh.I + 2 * sh.H * 2 * sh.Is)
    down = Tv * (sh.K * 2 * sh.I * sh.H + 2 * sh.Is * sh.H)
    return {"gemm_up_gate_recompute": up, "gemm_dgrad_down": down, "gemm_dgrad_up_gate": up,
            "gemm_wgrad_down": down, "gemm_wgrad_up_gate": up}


def cpu_baseline_backward(wl, d, dout, K, target_s):
    """The CPU oracle's backward as it stands, on a bounded sample of real
    tokens (every gradient's contribution of those tokens)."""
    import oracle
    pad = d["pad_mask"]
    valid = np.nonzero(pad == 0)[0]
    args = (d["w_router"], d["w13"], d["w2"], d["ws13"], d["ws2"])
    n, total_t = 0, 0.0
    while total_t < target_s and n < valid.size:
        rows = valid[n:n + 1]
        t0 = time.perf_counter()
        oracle.moe_backward(d["x"][rows], *args, dout[rows], K)
        total_t += time.perf_counter() - t0
        n += 1
    return {"value": n / total_t, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{n} real tokens of {wl.name} (all gradients, fp64 C, one thread), "
                      f"{total_t:.1f} s"}


def train_bench(args, m, wl, d, dd, pad, stream):
    """Times a training step of the layer: hi3_moe_forward_train (forward,
    keeping the routes, u, g, h) then hi3_moe_backward_after_forward (all six
    gradients without recomputing the forward)."""
    import torch
    sh = wl.shape
    dout_h = wk.make_dout(wl, args.seed)
    dout = torch.from_numpy(dout_h.view(np.int16)).cuda().view(torch.bfloat16) \
        if sh.dtype == wk.BF16 else torch.from_numpy(dout_h).cuda()
    x = dd["x"]
    dt = x.dtype
    out = torch.zeros_like(x)
    idx = torch.empty((wl.T, sh.K), dtype=torch.int32, device="cuda")
    wts = torch.empty((wl.T, sh.K), dtype=torch.float32, device="cuda")
    cnt = torch.empty((sh.E,), dtype=torch.int32, device="cuda")
    dx = torch.zeros_like(x)
    dwr = torch.empty((sh.E, sh.H), dtype=torch.float32, device="cuda")
    dw13 = torch.empty((sh.E, 2 * sh.I, sh.H), dtype=dt, device="cuda")
    dw2 = torch.empty((sh.E, sh.H, sh.I), dtype=dt, device="cuda")
    dws13 = torch.empty((2 * sh.Is, sh.H), dtype=dt, device="cuda")
    dws2 = torch.empty((sh.H, sh.Is), dtype=dt, device="cuda")
    n = m.hi3_moe_backward_workspace_size(wl.T, sh.H, sh.E, sh.K, sh.I, sh.Is,
                                          m.dtype_code(dt))
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    w = (dd["w_router"], dd["w13"], dd["w2"], dd["ws13"], dd["ws2"])

    def step():
        m.hi3_moe_forward_train(x, *w, pad, sh.K, out, idx, wts, cnt, ws, stream)
        m.hi3_moe_backward_after_forward(x, *w, pad, dout, sh.K, dx, dwr, dw13, dw2, dws13, dws2,
                                         ws, stream)

    hip = HipEvents()
    hip.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    ev = hip.create(3)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] {args.warmup} warmup steps done")
    fwd_ms = bwd_ms = 0.0
    t0 = time.perf_counter()
    for _ in range(args.steps):
        hip.hip.hipEventRecord(ev[0], ctypes.c_void_p(stream.cuda_stream))
        m.hi3_moe_forward_train(x, *w, pad, sh.K, out, idx, wts, cnt, ws, stream)
        hip.hip.hipEventRecord(ev[1], ctypes.c_void_p(stream.cuda_stream))
        m.hi3_moe_backward_after_forward(x, *w, pad, dout, sh.K, dx, dwr, dw13, dw2, dws13, dws2,
                                         ws, stream)
        hip.hip.hipEventRecord(ev[2], ctypes.c_void_p(stream.cuda_stream))
        fwd_ms += hip.elapsed_ms(ev[0], ev[1])
        bwd_ms += hip.elapsed_ms(ev[1], ev[2])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    hip.destroy(ev)
    log(f"[bench] {args.steps} timed steps done")
    ms_per_step = elapsed * 1e3 / args.steps
    gf = backward_gemm_flops(wl)
    # algorithmic FLOP of a training step: the forward's GEMMs and twice them
    flops = 3 * (gf["gemm_up_gate_recompute"] + gf["gemm_dgrad_down"])
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    line = {
        "metric": "MoE-layer training-step tokens/s (forward + all gradients), 64e top-8, "
                  "H=4096, 1 GPU",
        "value": round(wl.T_valid / (ms_per_step * 1e-3), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if sh.dtype == wk.BF16 else "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "entry": "train", "T": wl.T, "T_valid": wl.T_valid,
                   "H": sh.H, "E": sh.E, "K": sh.K, "I": sh.I, "I_shared": sh.Is,
                   "seed": args.seed},
        "tflops": round(tflops, 1), "frac_bf16_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "stages": {"forward_train": {"us": round(fwd_ms / args.steps * 1e3, 1)},
                   "backward_after_forward": {"us": round(bwd_ms / args.steps * 1e3, 1)}},
        "roofline": None, "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def backward_bench(args, m, wl, d, dd, pad, stream):
    """Times hi3_moe_backward per step (all six gradients), with per-stage
    HIP events; the roofline entry is the slowest GEMM stage."""
    import torch
    sh = wl.shape
    dout_h = wk.make_dout(wl, args.seed)
    dout = torch.from_numpy(dout_h.view(np.int16)).cuda().view(torch.bfloat16) \
        if sh.dtype == wk.BF16 else torch.from_numpy(dout_h).cuda()
    x = dd["x"]
    dt = x.dtype
    dx = torch.zeros_like(x)
    dwr = torch.empty((sh.E, sh.H), dtype=torch.float32, device="cuda")
    dw13 = torch.empty((sh.E, 2 * sh.I, sh.H), dtype=dt, device="cuda")
    dw2 = torch.empty((sh.E, sh.H, sh.I), dtype=dt, device="cuda")
    dws13 = torch.empty((2 * sh.Is, sh.H), dtype=dt, device="cuda")
    dws2 = torch.empty((sh.H, sh.Is), dtype=dt, device="cuda")
    n = m.hi3_moe_backward_workspace_size(wl.T, sh.H, sh.E, sh.K, sh.I, sh.Is,
                                          m.dtype_code(dt))
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    log(f"[bench] backward workspace {n / 2**20:.0f} MiB")

    def step(events=None):
        a = (x, dd["w_router"], dd["w13"], dd["w2"], dd["ws13"], dd["ws2"], pad, dout, sh.K,
             dx, dwr, dw13, dw2, dws13, dws2, ws)
        if events is None:
            m.hi3_moe_backward(*a, stream)
        else:
            m.hi3_moe_backward_instrumented(*a, events, stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] {args.warmup} warmup steps done")
    hip = HipEvents()
    ns = m.HI3_NUM_BWD_STAGES
    evsets = [hip.create(ns + 1) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evsets[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    log(f"[bench] {args.steps} timed steps done")
    stage_ms = np.zeros(ns)
    step_ms = []
    for evs in evsets:
        for k in range(ns):
            stage_ms[k] += hip.elapsed_ms(evs[k], evs[k + 1])
        step_ms.append(hip.elapsed_ms(evs[0], evs[ns]))
    stage_ms /= args.steps
    for evs in evsets:
        hip.destroy(evs)
    names = [m.hi3_moe_backward_stage_name(k) for k in range(ns)]
    ms_per_step = elapsed * 1e3 / args.steps
    gf = backward_gemm_flops(wl)
    stages = {}
    for k, name in enumerate(names):
        e = {"us": round(stage_ms[k] * 1e3, 2)}
        if name in gf and stage_ms[k] > 0:
            e["tflops"] = round(gf[name] / (stage_ms[k] * 1e-3) / 1e12, 1)
            e["frac_bf16_peak"] = round(e["tflops"] / PEAK_BF16_TFLOPS, 4)
        stages[name] = e
    for name, e in stages.items():
        log(f"  {name:24s} {e}")
    dom = max(gf, key=lambda k: stage_ms[names.index(k)])
    dom_ms = stage_ms[names.index(dom)]
    achieved = gf[dom] / (dom_ms * 1e-3) / 1e12
    mode = {"gemm_up_gate_recompute": 0, "gemm_dgrad_down": 2, "gemm_dgrad_up_gate": 3,
            "gemm_wgrad_down": 4, "gemm_wgrad_up_gate": 4}[dom]
    roofline = {"kernel": f"gemm_bf16_kernel<{mode}> ({dom})", "bound": "mfma",
                "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None}
    # algorithmic FLOP of the backward proper (twice the forward's GEMMs),
    # without the recomputed [up; gate] projection
    flops = sum(v for k, v in gf.items() if k != "gemm_up_gate_recompute")
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    cpu = None
    if args.cpu_seconds > 0:
        log("[bench] timing the CPU oracle's backward on a sample")
        cpu = cpu_baseline_backward(wl, d, dout_h, sh.K, args.cpu_seconds)
    line = {
        "metric": "MoE-layer backward tokens/s (all gradients), 64e top-8, H=4096, 1 GPU",
        "value": round(wl.T_valid / (ms_per_step * 1e-3), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if sh.dtype == wk.BF16 else "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "entry": "backward", "T": wl.T, "T_valid": wl.T_valid,
                   "H": sh.H, "E": sh.E, "K": sh.K, "I": sh.I, "I_shared": sh.Is,
                   "seed": args.seed},
        "tflops": round(tflops, 1), "frac_bf16_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "call_ms": {"median": round(float(np.median(step_ms)), 4),
                    "min": round(float(np.min(step_ms)), 4)},
        "stages": stages, "roofline": roofline, "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="image_1024", choices=wk.WORKLOADS)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="wall-time budget of the CPU oracle sample (0 = skip)")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip measuring the achievable peaks (probe, library GEMM, copy)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (counter calibration)")
    ap.add_argument("--entry", default="forward",
                    choices=("forward", "norm_residual", "backward", "train"),
                    help="forward: the layer (hi3_moe_forward); norm_residual: the layer "
                         "inside its block, h + layer(RMSNorm(h)) "
                         "(hi3_moe_forward_norm_residual); backward: all gradients of the "
                         "layer (hi3_moe_backward); train: hi3_moe_forward_train + "
                         "hi3_moe_backward_after_forward")
    args = ap.parse_args()
    if args.calibrate_copy:
        copy_calibration(args.calibrate_copy)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the layer is measured on one GPU's share)", file=sys.stderr)
        sys.exit(2)

    import torch
    import moe_decoder_ffn_amd as m

    wl = wk.workload(args.workload, args.seed)
    sh = wl.shape
    log(f"[bench] workload {wl.name}: T={wl.T} real={wl.T_valid} H={sh.H} E={sh.E} "
        f"K={sh.K} I={sh.I} Is={sh.Is}")
    t0 = time.perf_counter()
    d = wk.make_inputs(wl, args.seed)
    log(f"[bench] inputs generated in {time.perf_counter() - t0:.1f} s")

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(a).cuda()

    dd = {k: dev(v) for k, v in d.items()}
    pad = dd["pad_mask"] if wl.T != wl.T_valid else None
    x = dd["x"]
    out = torch.zeros_like(x)
    idx = torch.empty((wl.T, sh.K), dtype=torch.int32, device="cuda")
    wts = torch.empty((wl.T, sh.K), dtype=torch.float32, device="cuda")
    cnt = torch.empty((sh.E,), dtype=torch.int32, device="cuda")
    ws = m.workspace_for(x, sh.E, sh.K, sh.I, sh.Is)
    log(f"[bench] workspace {ws.numel() / 2**20:.0f} MiB")
    stream = torch.cuda.current_stream()
    # the caller's second stream for hi3_moe_forward_overlap (default priority)
    side_stream = torch.cuda.Stream()
    wargs = (dd["w_router"], dd["w13"], dd["w2"], dd["ws13"], dd["ws2"])

    def step(events=None, side=None):
        if events is None and side is None:
            m.hi3_moe_forward(x, *wargs, pad, sh.K, out, idx, wts, cnt, ws, stream=stream)
        elif events is None:
            m.hi3_moe_forward_overlap(x, *wargs, pad, sh.K, out, idx, wts, cnt, ws,
                                      side_stream=side, stream=stream)
        else:
            m.hi3_moe_forward_instrumented(x, *wargs, pad, sh.K, out, idx, wts, cnt, ws,
                                           events, stream=stream, side_stream=side)

    if args.entry == "norm_residual":
        norm_residual_bench(args, m, wl, d, dd, pad, ws, stream)
        return
    if args.entry in ("backward", "train"):
        del ws
        (backward_bench if args.entry == "backward" else train_bench)(args, m, wl, d, dd, pad,
                                                                     stream)
        return

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] {args.warmup} warmup steps done")

    hip = HipEvents()
    ns = m.HI3_NUM_STAGES
    names = [m.hi3_moe_stage_name(s) for s in range(ns)]
    dom = "gemm_up_gate_swiglu"
    di = names.index(dom)
    # timed steps: events only around the dominant kernel's stage (the
    # library skips NULL entries), so the timed calls carry two event records
    pairs = [hip.create(2) for _ in range(args.steps)]
    sparse = [[None] * di + pr + [None] * (ns - di - 1) for pr in pairs]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(sparse[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    log(f"[bench] {args.steps} timed steps done")
    dom_ms = sum(hip.elapsed_ms(a, b) for a, b in pairs) / args.steps
    for pr in pairs:
        hip.destroy(pr)

    def stage_pass(side):
        """As many calls as timed steps with every stage's events, after the
        timed region; returns per-stage ms and per-call ms."""
        evsets = [hip.create(ns + 1) for _ in range(args.steps)]
        torch.cuda.synchronize()
        for i in range(args.steps):
            step(evsets[i], side)
        torch.cuda.synchronize()
        st_ms = np.zeros(ns)
        call = []
        for evs in evsets:
            for k in range(ns):
                st_ms[k] += hip.elapsed_ms(evs[k], evs[k + 1])
            call.append(hip.elapsed_ms(evs[0], evs[ns]))
        for evs in evsets:
            hip.destroy(evs)
        return st_ms / args.steps, call

    # on one stream (the timed entry point), where every kernel has the GPU
    # to itself ...
    stage_ms, step_ms = stage_pass(None)
    log(f"[bench] {args.steps} per-stage steps done (one stream)")
    # ... and with the shared expert's GEMMs on the side stream where every
    # row is real (hi3_moe_forward_overlap): the grouped launches then hold
    # the routed rows alone and share the GPU with the dense launches
    side = m.hi3_moe_forward_shared_on_side(wl.T, sh.H, sh.E, sh.K, sh.I, sh.Is, sh.dtype,
                                            pad is not None)
    ov_ms, ov_call = stage_pass(side_stream)
    log(f"[bench] {args.steps} per-stage steps done (side stream)")

    ms_per_step = elapsed * 1e3 / args.steps
    tokens_s = wl.T_valid / (ms_per_step * 1e-3)
    flops = wl.T_valid * wk.flop_per_valid_token(sh)
    tflops = flops / (ms_per_step * 1e-3) / 1e12

    # one stream: the GEMM stages (and the dominant kernel) hold the routed
    # and the shared rows; beside the side stream, the routed rows alone
    gf = gemm_flops(wl, shared=True)
    gf_ov = gemm_flops(wl, shared=not side)
    sb = stage_bytes(wl)

    def stage_table(st_ms, g):
        out_ = {}
        for k, name in enumerate(names):
            e = {"us": round(st_ms[k] * 1e3, 2)}
            if name in g and st_ms[k] > 0:
                e["tflops"] = round(g[name] / (st_ms[k] * 1e-3) / 1e12, 1)
                e["frac_bf16_peak"] = round(e["tflops"] / PEAK_BF16_TFLOPS, 4)
            if name in sb and st_ms[k] > 0:
                e["gbs"] = round(sb[name] / (st_ms[k] * 1e-3) / 1e9, 1)
                e["frac_hbm"] = round(e["gbs"] / PEAK_HBM_GBS, 4)
            out_[name] = e
        return out_

    stages = stage_table(stage_ms, gf)
    stages_ov = stage_table(ov_ms, gf_ov)
    for name in names:
        log(f"  {name:22s} one stream: {stages[name]}  side stream: {stages_ov[name]}")

    kname = "gemm_bf16_kernel<0> (grouped [up; gate] + SwiGLU, routed and shared rows)"
    kname_ov = ("gemm_bf16_kernel<0> (routed rows alone, beside the shared expert's "
                "gemm_bf16_dense_kernel<0> on the side stream)" if side else kname)
    ui = names.index("gemm_up_gate_swiglu")
    wi = names.index("gemm_down")
    if sh.dtype == wk.BF16 and wl.T_valid * sh.K <= RIDGE_ROWS * sh.E:
        # few rows per expert: the weights are the traffic (HBM roofline)
        achieved = upgate_bytes(wl, shared=True) / (dom_ms * 1e-3) / 1e9
        roofline = {"kernel": kname, "bound": "hbm", "achieved": round(achieved, 1),
                    "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                    "traffic": measured_traffic(wl.name)}
        a_ov = upgate_bytes(wl, shared=not side) / (ov_ms[ui] * 1e-3) / 1e9
        roofline_ov = {"kernel": kname_ov, "achieved": round(a_ov, 1), "unit": "GB/s",
                       "frac": round(a_ov / PEAK_HBM_GBS, 4)}
    else:
        achieved = gf[dom] / (dom_ms * 1e-3) / 1e12
        roofline = {"kernel": kname, "bound": "mfma", "achieved": round(achieved, 1),
                    "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                    "traffic": measured_traffic(wl.name)}
        a_ov = gf_ov[dom] / (ov_ms[ui] * 1e-3) / 1e12
        roofline_ov = {"kernel": kname_ov, "achieved": round(a_ov, 1), "unit": "TFLOP/s",
                       "frac": round(a_ov / PEAK_BF16_TFLOPS, 4)}
    gemm_ms = stage_ms[ui] + stage_ms[wi]
    gemm_rate = sum(gf.values()) / (gemm_ms * 1e-3) / 1e12

    peaks = None
    if not args.no_peaks:
        log("[bench] measuring the achievable peaks")
        peaks = achievable_peaks(m)
    load = expert_load(to_np(cnt))

    cpu = None
    if args.cpu_seconds > 0:
        log("[bench] timing the CPU oracle on a sample")
        cpu = cpu_baseline(wl, d, sh.K, args.cpu_seconds)

    line = {
        "metric": METRIC, "value": round(tokens_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if sh.dtype == wk.BF16 else "f32", "data": "synthetic",
        "config": {"workload": wl.name, "entry": "forward", "T": wl.T,
                   "T_valid": wl.T_valid, "H": sh.H, "E": sh.E, "K": sh.K, "I": sh.I,
                   "I_shared": sh.Is, "seed": args.seed},
        "tflops": round(tflops, 1), "frac_bf16_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        # per call of the per-stage passes, first to last kernel on the stream
        # (HIP events); the dominant kernel's time (roofline) is the timed
        # steps' own: dominant_kernel_us
        "call_ms": {"median": round(float(np.median(step_ms)), 4),
                    "min": round(float(np.min(step_ms)), 4),
                    "overlap_median": round(float(np.median(ov_call)), 4)},
        "dominant_kernel_us": round(dom_ms * 1e3, 2),
        "stages": stages,
        "roofline": roofline,
        "gemms": {"us": round(gemm_ms * 1e3, 1), "tflops": round(gemm_rate, 1),
                  "frac_bf16_peak": round(gemm_rate / PEAK_BF16_TFLOPS, 4)},
        # hi3_moe_forward_overlap: the shared expert on the side stream
        "overlap": {"shared_on_side": bool(side), "stages": stages_ov,
                    "roofline": roofline_ov},
        "peaks": {"bf16_tflops": PEAK_BF16_TFLOPS, "hbm_gbs": PEAK_HBM_GBS,
                  "achievable": peaks},
        "expert_load": load,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def to_np(t):
    return t.cpu().numpy()


if __name__ == "__main__":
    main()
