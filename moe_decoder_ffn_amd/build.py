"""Builds libhi3moe.so (HIP, gfx950) in-tree with hipcc.

Each source is compiled separately (in parallel) and linked into one shared
library next to this file. Packed-fp32 VALU instructions are disabled for all
device code."""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libhi3moe.so")
SOURCES = ["router.hip", "dispatch.hip", "gemm.hip", "combine.hip", "norm.hip", "backward.hip",
           "hi3_moe.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC,
]


def _compile(src: str, verbose: bool, defines, build_dir) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *[f"-D{d}" for d in defines]]
    if src.endswith(".cpp"):
        cmd += ["-x", "hip"]
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        print(r.stderr, file=sys.stderr)
    return obj


def build(verbose: bool = False, defines=(), out: str = LIB) -> str:
    """defines: extra preprocessor definitions (e.g. GEMM tile settings),
    out: library path (default: next to this file)."""
    build_dir = BUILD if not defines else os.path.join(BUILD, "_".join(defines))
    os.makedirs(build_dir, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, defines, build_dir), SOURCES))
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", out + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
