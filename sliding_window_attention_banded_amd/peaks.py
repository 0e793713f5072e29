"""Achievable MFMA, LDS and HBM rates of the GPU (csrc/peaks.hip).

    python -m sliding_window_attention_banded_amd.peaks          # build and run
    python -m sliding_window_attention_banded_amd.peaks --build  # build only

The probe is a standalone HIP program; it measures the dense bf16 MFMA rate
with constant and with random operands (the sustained clock drops when the
operands toggle), the LDS read bandwidth per CU and the HBM copy bandwidth,
which put the published peaks of the roofline in context.
"""
from __future__ import annotations

import os
import subprocess
import sys

from .build import HIPCC_FLAGS, hipcc

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "csrc", "peaks.hip")
EXE = os.path.join(HERE, "peaks_probe")


def build(verbose: bool = False) -> str:
    flags = [f for f in HIPCC_FLAGS if f not in ("-shared", "-fPIC")]
    cmd = [hipcc(), *flags, SRC, "-o", EXE + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(EXE + ".tmp", EXE)
    return EXE


def run() -> str:
    if not os.path.exists(EXE):
        raise FileNotFoundError(f"{EXE} is missing: build it with "
                                "`python -m sliding_window_attention_banded_amd.peaks --build`")
    res = subprocess.run([EXE], check=True, capture_output=True, text=True)
    return res.stdout


if __name__ == "__main__":
    if "--build" in sys.argv[1:]:
        build(verbose=True)
        sys.exit(0)
    if not os.path.exists(EXE):
        build()
    sys.stdout.write(run())
