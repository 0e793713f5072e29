"""GPU parity of the backward pass: the HIP library's gradients against the
float64 oracle's, element by element, on the same bf16 inputs and cotangent.

The forward runs on the GPU first (its O and LSE are the backward's inputs,
as in training); the oracle recomputes everything from the inputs. Small and
ragged shapes are compared in full; the full-size workloads on whole
(batch, head) slices, which the oracle computes one at a time.

Tolerance: every element within a bound derived from the GPU path's
rounding and the magnitudes of the terms that make up that element
(tests/_bwd.py), so rows whose gradient cancels large terms get the room
their arithmetic needs and no more; plus relative RMS <= 1e-2 per tensor on
inputs without such cancellation.
"""
import pytest
import torch

from sliding_window_attention_banded_amd.workloads import (
    WORKLOADS, Workload, item_globals, make_inputs)
from tests._bwd import check_grads, cotangent, gpu_forward_backward
from tests._lib import ensure_library, to64

pytestmark = pytest.mark.gpu


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


@pytest.mark.parametrize("wl", SMALL, ids=lambda w: w.name)
@pytest.mark.parametrize("kind", ["normal", "sharp", "dedup"])
def test_backward_small(wl, kind):
    if kind == "dedup" and not any(len(g) for g in item_globals(wl)):
        pytest.skip("dedup inputs need global tokens")
    for seed in (0, 1):
        print(f"[bwd] {wl.name} B{wl.batch} H{wl.heads} n{wl.n} causal={wl.causal} "
              f"seed={seed} kind={kind}", flush=True)
        inp = make_inputs(wl, seed, kind)
        dout = cotangent(wl, seed)
        o, _, got = gpu_forward_backward(wl, inp, dout)
        ref = _oracle_grads(wl, inp, dout)
        check_grads(wl, inp, dout, o, got, ref, label=f"{wl.name}/{kind}/{seed}",
                    rel=None if kind == "dedup" else 1e-2)


FULL_SLICES = [
    ("encoder_b2_h12_n4096_w512", [(0, 0), (1, 11)]),
    ("encoder_b2_h12_n4096_w512_g1", [(0, 5), (1, 0)]),
    ("arlm_b1_h12_n8192_w512_causal_dil2", [(0, 3), (0, 11)]),
    # the 23,040-token stage: one head of dilation 1 and one of dilation 4
    ("arlm_b1_h8_n23040_w1024_causal_dil4", [(0, 0)]),
    ("arlm_b1_h8_n23040_w1024_causal_dil4", [(0, 7)]),
    ("qa_b4_h12_n4096_w512_g64", [(3, 7)]),
    ("qa_b4_h12_n4096_w512_gper", [(2, 1), (3, 5)]),
    # the LED encoder (16K tokens, one global token): its global-column
    # backward blocks take 4096 query positions each
    ("led_b1_h12_n16384_w1024_g1", [(0, 0)]),
    ("led_decoder_b1_h12_n1024_causal", [(0, 0), (0, 11)]),
]


@pytest.mark.parametrize("name,bh", FULL_SLICES,
                         ids=[f"{n}-{'-'.join(f'{b}.{h}' for b, h in bh)}" for n, bh in FULL_SLICES])
@pytest.mark.parametrize("kind", ["normal", "sharp", "dedup"])
def test_backward_full_size_slices(name, bh, kind):
    wl = WORKLOADS[name]
    if kind == "dedup" and not any(len(g) for g in item_globals(wl)):
        pytest.skip("dedup inputs need global tokens")
    print(f"[bwd] {wl.name} slices {bh} kind={kind}", flush=True)
    inp = make_inputs(wl, 0, kind)
    dout = cotangent(wl, 0)
    o, _, got = gpu_forward_backward(wl, inp, dout)
    refs = _oracle_grads(wl, inp, dout, bh=bh)
    check_grads(wl, inp, dout, o, got, refs, bh=bh, label=f"{wl.name}/{kind}",
                rel=None if kind == "dedup" else 1e-2)


# Long sequences with several global tokens: the global rows' gradients come
# from many key chunks and the global columns' from many query chunks
LONG_G_BWD = [
    Workload("long_globals_bwd", 1, 2, 9000, 64, (64, 128), (1, 2), False, (0, 4500, 8999), "bf16", 0.125),
    Workload("long_globals_bwd_causal", 1, 2, 9000, 64, (64, 128), (1, 2), True, (3, 4500, 8999), "bf16",
             0.125),
]


@pytest.mark.parametrize("wl", LONG_G_BWD, ids=lambda w: w.name)
@pytest.mark.parametrize("kind", ["normal", "dedup"])
def test_backward_long_sequence_globals(wl, kind):
    bh = [(0, 0), (0, 1)]
    print(f"[bwd] {wl.name} slices {bh} kind={kind}", flush=True)
    inp = make_inputs(wl, 0, kind)
    dout = cotangent(wl, 0)
    o, _, got = gpu_forward_backward(wl, inp, dout)
    refs = _oracle_grads(wl, inp, dout, bh=bh)
    check_grads(wl, inp, dout, o, got, refs, bh=bh, label=f"{wl.name}/{kind}",
                rel=None if kind == "dedup" else 1e-2)


def F(name, B, H, n, window, dilation, causal=False, G=()):
    win = (window,) * H if isinstance(window, int) else tuple(window)
    dil = (dilation,) * H if isinstance(dilation, int) else tuple(dilation)
    return Workload(name, B, H, n, 64, win, dil, causal, tuple(G), "fp32", 0.125)


# the fp32 path: the single-head fp32 shape of the benchmark configurations
# (n 512, window 64) and the same kinds of configuration as above
SMALL_F32 = [
    F("f_single_head", 1, 1, 512, 64, 1),
    F("f_mix_causal", 1, 3, 300, (32, 64, 2), (1, 2, 3), True),
    F("f_g", 2, 2, 257, (64, 16), (1, 3), False, (0, 100, 256)),
    F("f_g1_causal", 1, 2, 200, (32, 8), (2, 1), True, (120,)),
    F("f_per_item", 3, 2, 150, (16, 64), (1, 2), False, ((0, 5), (), (149,))),
    F("f_wide", 1, 2, 100, (400, 0), (1, 1)),
]


@pytest.mark.parametrize("wl", SMALL_F32, ids=lambda w: w.name)
@pytest.mark.parametrize("kind", ["normal", "sharp", "dedup"])
def test_backward_fp32(wl, kind):
    """fp32 gradients against the float64 oracle: the per-element bound with
    the rounding of fp32 sums (2^-20: a few units of 2^-24 over sums of up
    to a few thousand terms) in place of the bf16 operands' 2^-8, plus the
    rounding of the fp32 score and dP dot products (2^-21 = 8 units of 2^-24
    of sum_d |q_d k_d|: the six-level lane sum, the multiply, the
    exponential; tests/_bwd.py)."""
    if kind == "dedup" and not any(len(g) for g in item_globals(wl)):
        pytest.skip("dedup inputs need global tokens")
    print(f"[bwd-f32] {wl.name} B{wl.batch} H{wl.heads} n{wl.n} causal={wl.causal} kind={kind}",
          flush=True)
    inp = make_inputs(wl, 0, kind)
    dout = cotangent(wl, 0)
    o, _, got = gpu_forward_backward(wl, inp, dout)
    assert all(g is None or g.dtype == torch.float32 for g in got)
    ref = _oracle_grads(wl, inp, dout)
    check_grads(wl, inp, dout, o, got, ref, label=f"{wl.name}/{kind}",
                rel=None if kind == "dedup" else 1e-5, rnd=2.0 ** -20, serr=2.0 ** -21)
