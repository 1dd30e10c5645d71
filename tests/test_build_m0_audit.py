"""The build's check of the GEMM kernels' inline-asm copies (build.py,
audit_m0): in a kernel that issues them, M0 may only be written by the copy
sequence itself; any other use fails the build."""
import importlib.util
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
spec = importlib.util.spec_from_file_location(
    "_hi3_build", os.path.join(ROOT, "moe_decoder_ffn_amd", "build.py"))
build = importlib.util.module_from_spec(spec)
spec.loader.exec_module(build)

KERNEL = "0000000000004400 <_ZN3hi316gemm_bf16_kernelILi0ELi256ELi64ELi2ELi4ELi1EEEvNS_8GemmArgsE>:"
OTHER = "0000000000009900 <_ZN3hi314combine_kernelILi1ELi8EEEvNS_11CombineArgsE>:"
COPY = ["\ts_mov_b32 m0, s4  // 0000: BEFC0004", "\ts_nop 0", "\tglobal_load_lds_dwordx4 v[2:3], off"]


def text(*blocks):
    return "\n".join(line for b in blocks for line in b) + "\n"


def test_copy_sequences_pass_and_are_counted():
    body = [KERNEL, "\tv_mov_b32 v1, 0", *COPY, "\tds_read_b128 v[4:7], v1", *COPY,
            "\ts_mov_b32 m0, vcc_lo", "\ts_nop 0", "\tglobal_load_lds_dwordx4 v[8:9], off"]
    assert build.audit_m0(text(body)) == 3


@pytest.mark.parametrize("stray", ["\ts_mov_b32 m0, s7", "\ts_mov_b32 s5, m0",
                                   "\tv_readlane_b32 v1, v2, m0",
                                   "\tglobal_load_lds_dwordx4 v[2:3], off",
                                   "\ts_sendmsg sendmsg(MSG_INTERRUPT)"])
def test_other_m0_use_fails(stray):
    body = [KERNEL, *COPY, stray, "\ts_endpgm"]
    with pytest.raises(RuntimeError):
        build.audit_m0(text(body))


def test_kernels_without_the_copies_are_not_constrained():
    assert build.audit_m0(text([OTHER, "\ts_mov_b32 m0, s7", "\ts_endpgm"])) == 0
