"""Compile libattn.so (all HIP kernels + the C ABI) for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libattn.so")
SOURCES = ["attn_api.cpp", "append.hip", "decode.hip", "noalloc.hip", "prefill_bf16.hip", "prefill_f32.hip"]

# Packed-fp32 VALU forms are kept out of the code objects on purpose.
FLAGS = ["-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-shared",
         "-mllvm", "-amdgpu-mfma-vgpr-form",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


PEAKS = os.path.join(HERE, "attn_peaks")  # measured-ceiling program bench.py runs
PEAKS_FLAGS = ["-O3", "-std=c++17", "--offload-arch=gfx950",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall"]


def build(verbose: bool = False, extra: list[str] | None = None) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *FLAGS, *(extra or []), "-x", "hip", *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    ptmp = PEAKS + ".tmp"
    pcmd = [hipcc(), *PEAKS_FLAGS, os.path.join(HERE, "peaks.hip"), "-o", ptmp]
    if verbose:
        print(" ".join(pcmd), flush=True)
    subprocess.run(pcmd, check=True)
    os.replace(ptmp, PEAKS)
    return LIB


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
    print("built", LIB)
