"""Build libswattn.so (gfx950) in place with hipcc.

    python -m sliding_window_attention_banded_amd.build

The library lands next to this file; the Python binding loads it from there.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libswattn.so")
SOURCES = [os.path.join(HERE, "csrc", "swattn.hip")]
HEADERS = [os.path.join(ROOT, "include", "swattn.h"),
           os.path.join(HERE, "csrc", "kernels.hpp"),
           os.path.join(HERE, "csrc", "backward.hpp"),
           os.path.join(HERE, "csrc", "project.hpp")]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed-fp32 VALU instructions anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs: the softmax reads them directly
    # instead of copying them out of AGPRs
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    # no NaN canonicalisation in max/min (a NaN input gives a NaN output
    # either way; infinities are still honoured: masking relies on -inf)
    "-fno-honor-nans",
    # kernels whose leading arguments are scalars get them in SGPRs at wave
    # start (kernels that start with a struct argument preload nothing)
    "-mllvm", "-amdgpu-kernarg-preload-count=4",
    "-Wno-unused-command-line-argument",
]


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(verbose: bool = False) -> str:
    """Compile every HIP source into LIB (always recompiles)."""
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(HERE, "csrc"), *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
