"""Build tests/c_abi/swattn_c_demo (a plain C99 caller of libswattn.so) with
gcc against the HIP runtime; the library must be built first.

    python tests/c_abi/build_demo.py
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PKG = os.path.join(ROOT, "sliding_window_attention_banded_amd")
SRC = os.path.join(HERE, "swattn_c_demo.c")
EXE = os.path.join(HERE, "swattn_c_demo")


def build(verbose: bool = False) -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(rocm, "include"),
           SRC, "-o", EXE + ".tmp",
           "-L", PKG, "-lswattn", "-Wl,-rpath,$ORIGIN/../../sliding_window_attention_banded_amd",
           "-L", os.path.join(rocm, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(rocm, "lib")]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(EXE + ".tmp", EXE)
    return EXE


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
