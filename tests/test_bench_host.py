"""Host-side parts of bench.py that need no GPU: the one-GPU guard, the
algorithmic FLOP and byte counts its roofline divides by (against the
layer's definition written out by hand for image_1024), the gate that
reports the committed HBM traffic only while the GEMM source matches it,
and the per-expert load summary."""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads as wk  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_gemm_flops_image_1024():
    wl = wk.workload("image_1024")
    T, H, K, I, Is = 4131, 4096, 8, 3072, 3072
    # [up; gate]: each routed row against 2I weight rows of H, the shared
    # row against 2 Is; down: I (Is) against H; 2 FLOP per multiply-add
    up = T * (K * 2 * H * 2 * I + 2 * H * 2 * Is)
    down = T * (K * 2 * I * H + 2 * Is * H)
    f = bench.gemm_flops(wl, shared=True)
    assert f == {"gemm_up_gate_swiglu": up, "gemm_down": down}
    fr = bench.gemm_flops(wl, shared=False)
    assert fr == {"gemm_up_gate_swiglu": T * K * 2 * H * 2 * I,
                  "gemm_down": T * K * 2 * I * H}


def test_upgate_bytes_image_1024():
    wl = wk.workload("image_1024")
    T, H, E, K, I, Is = 4131, 4096, 64, 8, 3072, 3072
    weights = (E * 2 * I * H + 2 * Is * H) * 2
    x_rows = T * (K + 1) * H * 2
    h_out = T * (K * I + Is) * 2
    assert bench.upgate_bytes(wl, shared=True) == weights + x_rows + h_out
    # the committed traffic summary states the same algorithmic bytes
    kv = {}
    with open(os.path.join(ROOT, "profiles",
                           "traffic_gemm_up_gate_swiglu_image_1024.txt")) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
    assert int(kv["algorithmic_read_bytes"]) == weights + x_rows
    assert int(kv["algorithmic_write_bytes"]) == h_out


def test_traffic_reported_only_for_the_committed_source(monkeypatch):
    path = os.path.join(ROOT, "profiles", "traffic_gemm_up_gate_swiglu_image_1024.txt")
    with open(path) as f:
        h = [ln.split("=", 1)[1].strip() for ln in f if ln.startswith("kernel_source_sha256")][0]
    monkeypatch.setattr(bench, "gemm_source_hash", lambda: h)
    t = bench.measured_traffic("image_1024")
    assert isinstance(t, int) and t > bench.upgate_bytes(wk.workload("image_1024"))
    assert bench.measured_traffic("prompt_512") is None  # no summary for it
    monkeypatch.setattr(bench, "gemm_source_hash", lambda: "0" * 64)
    assert bench.measured_traffic("image_1024") is None


def test_expert_load_summary():
    cnt = np.array([10, 10, 0, 20], dtype=np.int32)
    s = bench.expert_load(cnt)
    assert s == {"max_over_mean": 2.0, "min": 0, "max": 20, "experts_below_1pct_of_mean": 1}


@pytest.mark.parametrize("name", ["image_1024", "batch8_512", "prompt_512"])
def test_stage_bytes_are_the_stated_streams(name):
    wl = wk.workload(name)
    sh = wl.shape
    b = bench.stage_bytes(wl)
    Tv, H, E, K = wl.T_valid, sh.H, sh.E, sh.K
    assert b["router"] == Tv * H * 2 + E * H * 4 + wl.T * K * 8
    assert b["combine"] == Tv * (K * H * 4 + H * 4 + H * 2 + K * 8)
