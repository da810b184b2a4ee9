"""The inline-assembly hazard check (causal_linear_attention_chunked_amd/asm_check.py) that the
build runs: the scan itself on planted listings, and the library's sources as built.

A VALU write of an SGPR needs five wait states before a vector memory instruction reads that
SGPR; the compiler inserts them for its own instructions but not for inline assembly.  A listing
with a spilled buffer descriptor restored by v_readlane right before an inline LDS-direct load
faulted the GPU; the check flags exactly that sequence.
"""
import os
import shutil

import pytest

from causal_linear_attention_chunked_amd import asm_check, build

LOAD = "buffer_load_dword v6, s[8:11], 0 offen lds"


def block(*ins):
    return "\n".join(ins) + "\n"


def test_the_scan_flags_a_descriptor_written_just_before_an_inline_load():
    bad = block("v_readlane_b32 s11, v222, 16", ";;#ASMSTART", LOAD, ";;#ASMEND")
    assert len(asm_check.hazards(bad)) == 1


def test_the_scan_counts_wait_states():
    near = block("v_readfirstlane_b32 s9, v1", "s_nop 2", ";;#ASMSTART", LOAD, ";;#ASMEND")  # 3 + ... < 5
    far = block("v_readfirstlane_b32 s9, v1", "s_nop 4", ";;#ASMSTART", LOAD, ";;#ASMEND")   # 5
    apart = block("v_readlane_b32 s8, v2, 0", *(["s_add_u32 s0, s0, 1"] * 5), ";;#ASMSTART", LOAD, ";;#ASMEND")
    assert len(asm_check.hazards(near)) == 1
    assert asm_check.hazards(far) == [] and asm_check.hazards(apart) == []


def test_the_scan_ignores_other_registers_and_compiler_loads():
    other = block("v_readlane_b32 s12, v222, 16", ";;#ASMSTART", LOAD, ";;#ASMEND")  # s12 not read
    salu = block("s_mov_b32 s11, s3", ";;#ASMSTART", LOAD, ";;#ASMEND")              # SALU write: no hazard
    compiled = block("v_readlane_b32 s11, v222, 16", LOAD)  # outside assembly: the compiler's own
    assert asm_check.hazards(other) == [] and asm_check.hazards(salu) == [] and asm_check.hazards(compiled) == []


@pytest.mark.skipif(not os.path.exists(build.HIPCC) and not shutil.which(build.HIPCC), reason="hipcc not available")
def test_the_library_sources_have_no_hazard():
    flags = [f for f in build.DEVICE_FLAGS if f != "-fPIC"]
    assert asm_check.check(build.HIPCC, flags, build.CSRC) == []
