"""Build the HIP library ``libkvq.so`` in place with hipcc for gfx950.

Every kernel file is compiled with -O3 for gfx950 with packed-fp32 code
generation switched off; the append kernel additionally with
-ffp-contract=off, because its results must match a plain IEEE definition bit
for bit.  Run as ``python -m bit_kv_cache_quant_amd._build``.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libkvq.so")
OBJDIR = os.path.join(HERE, "_build")

SOURCES = {
    "kvq_api.hip": [],
    "append.hip": ["-ffp-contract=off"],
    # MFMA results straight into VGPRs (no accumulator-register copies)
    "decode_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "decode_f16_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "decode_grouped.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "prefill_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "combine.hip": [],
}

COMMON = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-function"]


def hipcc() -> str:
    for cand in ("/opt/rocm/bin/hipcc", "hipcc"):
        if os.path.sep not in cand or os.path.exists(cand):
            return cand
    return "hipcc"


def build(verbose: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    objs = []
    for src, extra in SOURCES.items():
        obj = os.path.join(OBJDIR, src.replace(".hip", ".o"))
        cmd = [hipcc(), "-c", os.path.join(CSRC, src), "-o", obj] + COMMON + extra
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
