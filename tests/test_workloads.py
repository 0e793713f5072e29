"""Seeded input generator and closed-form accounting (host logic only)."""
import numpy as np
import torch

from sliding_window_attention_banded_amd.accounting import (
    algorithmic_bytes, band_flops, useful_flops)
from sliding_window_attention_banded_amd.workloads import WORKLOADS, make_inputs


def test_inputs_are_seeded_and_shaped():
    wl = WORKLOADS["single_head_fp32_n512_w64"]
    a = make_inputs(wl, 0)
    b = make_inputs(wl, 0)
    c = make_inputs(wl, 1)
    assert a["q"].shape == (1, 1, 512, 64) and a["q"].dtype == torch.float32
    assert torch.equal(a["q"], b["q"]) and not torch.equal(a["q"], c["q"])
    assert a["qg"] is None
    assert abs(a["v"].std().item() - 8 ** -0.5) < 0.01


def test_bf16_inputs_round_to_nearest_even():
    wl = WORKLOADS["encoder_b2_h12_n4096_w512_g1"].with_(batch=1, heads=1, n=64)
    x = make_inputs(wl, 3)
    assert x["q"].dtype == torch.bfloat16 and x["kg"].shape == (1, 1, 64, 64)
    gen = torch.Generator().manual_seed(3)
    q32 = torch.randn((1, 1, 64, 64), generator=gen) * 0.125
    assert torch.equal(x["q"], q32.to(torch.bfloat16))


def test_sharp_and_dedup_kinds():
    wl = WORKLOADS["qa_b4_h12_n4096_w512_g64"].with_(batch=1, heads=1, n=256)
    s = make_inputs(wl, 0, "sharp")
    assert s["v"].float().abs().max() <= 1.0 and s["q"].float().std() > 1.5
    d = make_inputs(wl, 0, "dedup")
    assert (d["v"][0, 0, [0, 16, 32, 48]].float().sum(-1) == 1.0).all()
    assert torch.equal(d["k"][0, 0, 0], d["k"][0, 0, 16])


def test_accounting_matches_hand_counts():
    # encoder n=4096, w=512: interior rows have 513 keys; 256 rows at each end
    # lose 1..256 keys -> sum = 4096*513 - 2*(256*257/2)
    wl = WORKLOADS["encoder_b2_h12_n4096_w512"]
    keys = 4096 * 513 - 2 * (256 * 257 // 2)
    assert band_flops(wl) == 4 * 64 * 2 * 12 * keys
    assert abs(band_flops(wl) / 1e9 - 12.506) < 1e-3
    assert useful_flops(wl) == band_flops(wl)
    assert algorithmic_bytes(wl, with_lse=False) == 4 * 24 * 4096 * 64 * 2
    # causal, dilation 2 on two heads: each residue row keeps <= 257 keys
    wl3 = WORKLOADS["arlm_b1_h12_n8192_w512_causal_dil2"]
    assert abs(band_flops(wl3) / 1e9 - 6.350) < 1e-3
    wl4 = WORKLOADS["arlm_b1_h8_n23040_w1024_causal_dil4"]
    assert abs(band_flops(wl4) / 1e9 - 23.736) < 1e-3
    wl5 = WORKLOADS["qa_b4_h12_n4096_w512_g64"]
    assert abs(useful_flops(wl5) / 1e9 - 31.000) < 2e-3
    assert np.isclose(band_flops(wl5) / 1e9, 25.012, atol=1e-3)
