"""Host-side checks of the benchmark's command line and of its input sets
(no GPU): a request for more than one GPU ends with a message and a non-zero
status before anything touches a device, and the device input generator
draws the distributions it names."""
import subprocess
import sys
from dataclasses import replace
from pathlib import Path

import torch

from sliding_window_attention_banded_amd.workloads import WORKLOADS, Workload, make_device_inputs

ROOT = Path(__file__).resolve().parents[1]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_device_inputs_normal_and_sharp_on_cpu():
    wl = Workload("dev_inputs", 2, 3, 257, 64, (32, 16, 8), (1, 2, 1), False, (0, 100), "bf16", 0.125)
    a = make_device_inputs(wl, 5, "cpu", kind="normal")
    b = make_device_inputs(wl, 5, "cpu", kind="normal")
    for r in ("q", "k", "v", "qg", "kg", "vg"):
        assert a[r].shape == (2, 3, 257, 64) and a[r].dtype == torch.bfloat16
        assert torch.equal(a[r], b[r])  # seeded
        std = a[r].float().std().item()
        assert abs(std - 0.125) < 0.01, (r, std)
    s = make_device_inputs(wl, 5, "cpu", kind="sharp")
    assert s["v"].float().abs().max() <= 1.0 and s["q"].float().std() > 1.5
    nog = make_device_inputs(replace(WORKLOADS["encoder_b2_h12_n4096_w512"], n=64), 0, "cpu", "normal")
    assert nog["qg"] is None and nog["kg"] is None and nog["vg"] is None
