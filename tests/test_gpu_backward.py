"""GPU parity of the backward pass: the HIP library's gradients against the
float64 oracle's, element by element, on the same bf16 inputs and cotangent.

The forward runs on the GPU first (its O and LSE are the backward's inputs,
as in training); the oracle recomputes everything from the inputs. Small and
ragged shapes are compared in full; the full-size workloads on whole
(batch, head) slices, which the oracle computes one at a time.

Tolerance (bf16 gradients, fp32 accumulation): relative RMS <= 1e-2 and
max-abs <= 2^-5 * max|reference| per tensor. The terms: dS is rounded to
bf16 before its MFMA (relative 2^-8 per element), D_i is formed from the
bf16-rounded O (relative 2^-9), P and dP are fp32, and the gradients are
rounded to bf16 at the end (relative 2^-9 of each element). Summed over a
row's keys with random signs the first term stays near 2^-8 of the row's
largest contributions; 2^-5 of the tensor's largest element leaves room for
rows whose gradient is a cancellation of larger terms. A tensor that
vanishes exactly (window 0: every row's softmax is a single weight 1, so
dS = 0 and dq = dk = 0) is held to an absolute 1e-6, the fp32 rounding of
its O(1) terms.
"""
import numpy as np
import pytest
import torch

from sliding_window_attention_banded_amd.workloads import (
    WORKLOADS, Workload, item_globals, make_inputs)
from tests._lib import ensure_library, to64

pytestmark = pytest.mark.gpu

REL, MAXF, FLOOR = 1e-2, 2.0 ** -5, 1e-6


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_library()


def W(name, B, H, n, window, dilation, causal=False, G=()):
    win = (window,) * H if isinstance(window, int) else tuple(window)
    dil = (dilation,) * H if isinstance(dilation, int) else tuple(dilation)
    return Workload(name, B, H, n, 64, win, dil, causal, tuple(G), "bf16", 0.125)


SMALL = [
    W("b_uniform", 1, 2, 300, 64, 1),
    W("b_uniform_causal", 1, 2, 300, 64, 2, True),
    W("b_mix", 2, 3, 777, (64, 128, 30), (1, 2, 3)),
    W("b_mix_causal", 1, 4, 500, (32, 256, 2, 1024), (1, 4, 1, 2), True),
    W("b_short", 1, 2, 40, 16, 1),
    W("b_one", 1, 1, 1, 8, 1),
    W("b_wide", 1, 2, 200, (1000, 602), (1, 1)),
    W("b_window0", 1, 2, 130, (0, 0), (1, 5)),
    W("b_g1", 2, 2, 300, 64, 1, False, (0,)),
    W("b_g_mix", 2, 3, 777, (64, 128, 30), (1, 2, 3), False, (0, 17, 400, 776)),
    W("b_g_causal", 1, 4, 500, (32, 256, 2, 1024), (1, 4, 1, 2), True, (5, 250, 499)),
    W("b_g_many", 1, 2, 700, (64, 16), (1, 3), False, tuple(range(0, 700, 7))),
    W("b_g_all", 1, 2, 130, (8, 4), (1, 2), False, tuple(range(130))),
    W("b_per_item", 3, 2, 500, (64, 16), (1, 3), False, ((0, 5, 499), (), tuple(range(100, 190)))),
    W("b_per_item_causal", 2, 3, 400, (32, 256, 2), (1, 4, 1), True, ((7,), (0, 250, 399))),
    # one global token per item (its column folded in from registers): in
    # the middle (inside some rows' bands), dilated heads, causal, per item
    W("b_g1_mid_dil", 2, 3, 777, (64, 128, 30), (1, 2, 3), False, (401,)),
    W("b_g1_causal_dil", 1, 4, 500, (32, 256, 2, 1024), (1, 4, 1, 2), True, (250,)),
    W("b_g1_per_item", 3, 2, 500, (64, 16), (1, 3), False, ((5,), (), (499,))),
]

GRADS = ("dq", "dk", "dv", "dqg", "dkg", "dvg")


def _cotangent(wl, seed):
    g = torch.Generator().manual_seed(10_000 + seed)
    return torch.randn((wl.batch, wl.heads, wl.n, wl.d), generator=g).to(torch.bfloat16)


def _gpu_grads(wl, inp, dout):
    from sliding_window_attention_banded_amd import Plan
    dev = {k: (v.cuda() if v is not None else None) for k, v in inp.items()}
    with Plan(wl.batch, wl.heads, wl.n, wl.d, wl.window, wl.dilation, wl.causal,
              wl.global_idx, wl.torch_dtype) as pl:
        o, lse = pl.forward(dev["q"], dev["k"], dev["v"], dev["qg"], dev["kg"], dev["vg"],
                            want_lse=True)
        grads = pl.backward(dev["q"], dev["k"], dev["v"], o, lse, dout.cuda(),
                            dev["qg"], dev["kg"], dev["vg"])
        torch.cuda.synchronize()
    return [None if t is None else t.cpu() for t in grads]


def _oracle_grads(wl, inp, dout, bh=None):
    """Oracle gradients, optionally for a list of (b, h) slices only."""
    from oracle import attention_backward
    t = [to64(inp[k]) for k in ("q", "k", "v", "qg", "kg", "vg")] + [to64(dout)]
    win, dil = list(wl.window), list(wl.dilation)
    if bh is None:
        return attention_backward(*t, window=win, dilation=dil, causal=wl.causal,
                                  global_idx=list(wl.global_idx))
    outs = []
    for b, h in bh:
        sl = [None if x is None else x[b:b + 1, h:h + 1] for x in t]
        outs.append(attention_backward(*sl, window=win[h], dilation=dil[h], causal=wl.causal,
                                       global_idx=list(item_globals(wl)[b])))
    return outs


def _cmp(got, ref, label):
    g = got.double().numpy()
    assert np.isfinite(g).all(), f"{label}: non-finite gradient"
    err = np.abs(g - ref)
    scale = max(np.abs(ref).max(), 1e-30)
    rel = np.sqrt((err ** 2).mean()) / max(np.sqrt((ref ** 2).mean()), 1e-30)
    print(f"  {label}: max-abs {err.max():.3e} (max|ref| {scale:.3e}), rel-rms {rel:.3e}", flush=True)
    assert err.max() <= max(MAXF * scale, FLOOR), f"{label}: max-abs {err.max():.3e} > {MAXF} * {scale:.3e}"
    if np.sqrt((ref ** 2).mean()) > FLOOR:
        assert rel <= REL, f"{label}: rel-rms {rel:.3e}"


@pytest.mark.parametrize("wl", SMALL, ids=lambda w: w.name)
@pytest.mark.parametrize("kind", ["normal", "sharp"])
def test_backward_small(wl, kind):
    for seed in (0, 1):
        print(f"[bwd] {wl.name} B{wl.batch} H{wl.heads} n{wl.n} causal={wl.causal} "
              f"seed={seed} kind={kind}", flush=True)
        inp = make_inputs(wl, seed, kind)
        dout = _cotangent(wl, seed)
        got = _gpu_grads(wl, inp, dout)
        ref = _oracle_grads(wl, inp, dout)
        for name, a, b in zip(GRADS, got, ref):
            if b is None:
                assert a is None
                continue
            _cmp(a, b, f"{wl.name}/{kind}/{seed}/{name}")


@pytest.mark.parametrize("name,bh", [
    ("encoder_b2_h12_n4096_w512", [(0, 0), (1, 11)]),
    ("encoder_b2_h12_n4096_w512_g1", [(0, 5), (1, 0)]),
    ("arlm_b1_h12_n8192_w512_causal_dil2", [(0, 3), (0, 11)]),
    ("qa_b4_h12_n4096_w512_g64", [(3, 7)]),
    ("qa_b4_h12_n4096_w512_gper", [(2, 1), (3, 5)]),
    ("led_decoder_b1_h12_n1024_causal", [(0, 0), (0, 11)]),
])
@pytest.mark.parametrize("kind", ["normal", "sharp"])
def test_backward_full_size_slices(name, bh, kind):
    wl = WORKLOADS[name]
    print(f"[bwd] {wl.name} slices {bh} kind={kind}", flush=True)
    inp = make_inputs(wl, 0, kind)
    dout = _cotangent(wl, 0)
    got = _gpu_grads(wl, inp, dout)
    refs = _oracle_grads(wl, inp, dout, bh=bh)
    for (b, h), ref in zip(bh, refs):
        for name_g, a, r in zip(GRADS, got, ref):
            if r is None:
                continue
            _cmp(a[b:b + 1, h:h + 1], r, f"{wl.name}[{b},{h}]/{kind}/{name_g}")


def test_backward_rejects_fp32_plans():
    from sliding_window_attention_banded_amd import Plan, SwattnError
    x = torch.zeros((1, 1, 64, 64), dtype=torch.float32, device="cuda")
    lse = torch.zeros((1, 1, 64), dtype=torch.float32, device="cuda")
    with Plan(1, 1, 64, 64, 8, 1, False, (), torch.float32) as pl:
        with pytest.raises(SwattnError):
            pl.backward(x, x, x, x, lse, x)
