"""The C ABI from plain C: tests/c_abi/swattn_c_demo.c (C99, linked against
libswattn.so and the HIP runtime; no Python, no torch) rejects bad
parameters on the host, and runs a forward whose output matches the float64
oracle. Inputs and outputs cross as raw files."""
import os
import subprocess

import numpy as np
import pytest
import torch

from sliding_window_attention_banded_amd.workloads import Workload, make_inputs
from tests._lib import compare, ensure_library, oracle_ref

HERE = os.path.dirname(os.path.abspath(__file__))
EXE = os.path.join(HERE, "c_abi", "swattn_c_demo")


@pytest.fixture(scope="module")
def demo():
    ensure_library()
    if not os.path.exists(EXE):
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "build_demo", os.path.join(HERE, "c_abi", "build_demo.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()
    return EXE


def test_c_caller_gets_host_side_errors(demo):
    res = subprocess.run([demo, "validate"], capture_output=True, text=True, timeout=60)
    assert res.returncode == 0, res.stderr
    assert "validate: ok" in res.stdout


@pytest.mark.gpu
@pytest.mark.parametrize("causal,G", [(False, (0, 77, 299)), (True, ())])
def test_c_caller_forward_matches_oracle(demo, tmp_path, causal, G):
    H, n, w, dil = 2, 300, 64, 2
    wl = Workload("c_abi", 1, H, n, 64, (w,) * H, (dil,) * H, causal, G, "bf16")
    print(f"[c-abi] n{n} H{H} w{w} dil{dil} causal={causal} G={G}", flush=True)
    inp = make_inputs(wl, 0, "sharp")
    for name in ("q", "k", "v", "qg", "kg", "vg"):
        if inp[name] is not None:
            inp[name].contiguous().view(torch.int16).numpy().tofile(str(tmp_path / f"{name}.bin"))
    args = [demo, "run", str(tmp_path), "1", str(H), str(n), str(w), str(dil), str(int(causal))]
    args += [str(g) for g in G] if G else ["-1"]
    res = subprocess.run(args, capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stderr
    o = torch.from_numpy(np.fromfile(str(tmp_path / "o.bin"), dtype=np.int16)).view(torch.bfloat16)
    lse = torch.from_numpy(np.fromfile(str(tmp_path / "lse.bin"), dtype=np.float32))
    o = o.reshape(1, H, n, 64)
    lse = lse.reshape(1, H, n)
    ref_o, ref_lse = oracle_ref(wl, inp)
    compare(wl, o, lse, ref_o, ref_lse, label="c-abi")
