"""Builds libhi3moe.so (HIP, gfx950) in-tree with hipcc.

Each source is compiled separately (in parallel) and linked into one shared
library next to this file. Packed-fp32 VALU instructions are disabled for all
device code.

Compiler warnings are never hidden: every warning is printed, except the one
kind the GEMM source produces on purpose (an inline-asm clobber of M0, the
register that holds the LDS base of a direct global -> LDS copy), which is
counted and checked instead: after compiling, the gfx950 code object of
gemm.hip is disassembled and the build fails if, in a kernel that issues
those copies as inline assembly, anything other than that three-instruction
sequence reads or writes M0.
"""
import os
import re
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libhi3moe.so")
SOURCES = ["router.hip", "dispatch.hip", "gemm.hip", "combine.hip", "norm.hip", "backward.hip",
           "probe.hip", "noalloc.hip", "hi3_moe.cpp"]

ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.environ.get("HIPCC", os.path.join(ROCM, "bin", "hipcc"))
LLVM_BIN = os.path.join(ROCM, "llvm", "bin")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC,
]

# The M0 clobber warning of the inline-asm copies, and the note hipcc's host
# pass prints for the device-only target feature above.
M0_WARNING = "inline asm clobber list contains reserved registers: m0"
IGNORED_NOISE = ("'-packed-fp32-ops' is not a recognized feature for this target",
                 "warnings generated when compiling for")
# Kernels of gemm.hip that issue their copies as inline assembly: every
# bf16 grouped and dense GEMM.
ASM_COPY_KERNEL = re.compile(r"gemm_bf16_(dense_)?kernelILi\d+E")
# Instructions that use M0 without naming it.
IMPLICIT_M0 = re.compile(r"^(s_sendmsg|s_movrel|v_movrel|s_set_gpr_idx|ds_gws|ds_append|"
                         r"ds_consume|ds_ordered_count|v_interp)|(^|_)lds(_|$)")


def _filter_warnings(src: str, stderr: str):
    """Returns (M0 warnings counted, lines of every other diagnostic). A
    diagnostic is a warning or error line with the notes, source lines and
    carets that follow it."""
    m0 = 0
    other = []
    keep = True
    for line in stderr.splitlines():
        if re.search(r": (warning|error|fatal error): ", line):
            keep = M0_WARNING not in line
            if not keep:
                m0 += 1
        elif re.match(r"^\d+ warnings? generated", line.strip()) or \
                any(n in line for n in IGNORED_NOISE) or not line.strip():
            continue
        if keep:
            other.append(line)
    return m0, other


def check_m0(obj: str) -> int:
    """Disassembles the gfx950 code object inside obj (a hipcc object of this
    build) and checks that in every kernel issuing inline-asm copies, each
    M0 access is the copy sequence `s_mov_b32 m0, sN; s_nop 0;
    global_load_lds_dwordx4`. Returns the number of sequences checked;
    raises RuntimeError on any other use."""
    with tempfile.TemporaryDirectory() as tmp:
        fat = os.path.join(tmp, "fatbin")
        co = os.path.join(tmp, "gfx950.co")
        subprocess.run([os.path.join(LLVM_BIN, "llvm-objcopy"), f"--dump-section=.hip_fatbin={fat}",
                        obj, os.path.join(tmp, "copy.o")], check=True, capture_output=True)
        subprocess.run([os.path.join(LLVM_BIN, "clang-offload-bundler"), "--unbundle", "--type=o",
                        f"--input={fat}", "--targets=hipv4-amdgcn-amd-amdhsa--gfx950",
                        f"--output={co}"], check=True, capture_output=True)
        dis = subprocess.run([os.path.join(LLVM_BIN, "llvm-objdump"), "-d", "--mcpu=gfx950", co],
                             check=True, capture_output=True, text=True).stdout
    return audit_m0(dis)


def audit_m0(dis: str) -> int:
    """The M0 check of check_m0 on llvm-objdump -d text. Returns the number
    of copy sequences; raises RuntimeError on any other M0 use in a kernel
    that issues the inline-asm copies."""
    checked = 0
    func = None
    insts = []

    def audit(name, body):
        nonlocal checked
        if name is None or not ASM_COPY_KERNEL.search(name):
            return
        ops = [b.split("//")[0].strip() for b in body]
        i = 0
        while i < len(ops):
            op = ops[i]
            if re.match(r"s_mov_b32 m0, (s\d+|vcc_lo|vcc_hi|ttmp\d+)$", op):
                if (i + 2 < len(ops) and ops[i + 1] == "s_nop 0" and
                        ops[i + 2].startswith("global_load_lds_dwordx4")):
                    checked += 1
                    i += 3
                    continue
                raise RuntimeError(f"{name}: M0 written outside the copy sequence: {op}")
            if re.search(r"\bm0\b", op) or IMPLICIT_M0.search(op.split(" ")[0]):
                raise RuntimeError(f"{name}: instruction using M0 outside the copy sequence: {op}")
            i += 1

    for line in dis.splitlines():
        m = re.match(r"^[0-9a-f]+ <(\S+)>:$", line)
        if m:
            audit(func, insts)
            func, insts = m.group(1), []
        elif line.startswith("\t") and func is not None:
            insts.append(line.strip())
    audit(func, insts)
    return checked


def _compile(src: str, verbose: bool, defines, build_dir):
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
    m0, other = _filter_warnings(src, r.stderr)
    return obj, m0, other


def build(verbose: bool = False, defines=(), out: str = LIB) -> str:
    """defines: extra preprocessor definitions (e.g. GEMM tile settings),
    out: library path (default: next to this file)."""
    build_dir = BUILD if not defines else os.path.join(BUILD, "_".join(defines))
    os.makedirs(build_dir, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        results = list(ex.map(lambda s: _compile(s, verbose, defines, build_dir), SOURCES))
    objs = [r[0] for r in results]
    for src, (_, m0, other) in zip(SOURCES, results):
        for line in other:
            print(f"[hipcc {src}] {line}", file=sys.stderr)
        if m0:
            n = check_m0(os.path.join(build_dir, os.path.splitext(src)[0] + ".o"))
            print(f"[build] {src}: {m0} inline-asm M0 clobber warnings (the GEMMs' "
                  f"direct-to-LDS copies); disassembly checked: {n} copy sequences, no other "
                  "M0 use in those kernels", file=sys.stderr)
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", out + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
