"""Builds liblachunk.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

    python -m causal_linear_attention_chunked_amd.build
"""
from __future__ import annotations

import importlib.util
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "liblachunk.so")
SOURCES = ["la_api.cpp", "la_fwd.hip", "la_fwd2.hip", "la_bwd.hip", "la_bwd4.hip", "la_bwd_seq128.hip", "la_ce.hip", "la_fwd_seq128.hip",
           "la_cumsum.hip",
           "la_floor.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed-fp32 VALU ops are disabled for every device compile (the compiler forms
# them from ordinary float code otherwise).
DEVICE_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(verbose: bool = False) -> str:
    objs = []
    os.makedirs(os.path.join(HERE, "_build"), exist_ok=True)
    for src in SOURCES:
        obj = os.path.join(HERE, "_build", os.path.splitext(src)[0] + ".o")
        cmd = [HIPCC, *DEVICE_FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        objs.append(obj)
    # the inline-assembly check on the device assembly (the device flags; -fPIC is for the host)
    spec = importlib.util.spec_from_file_location("lachunk_asm_check", os.path.join(HERE, "asm_check.py"))
    asm_check = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(asm_check)
    found = asm_check.check(HIPCC, [f for f in DEVICE_FLAGS if f != "-fPIC"], CSRC)
    if found:
        raise RuntimeError("inline assembly too close to a VALU write of its SGPRs:\n" + "\n".join(found))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
