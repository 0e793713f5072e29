"""The per-element backward bound of tests/_bwd.py, checked on the CPU.

1. It covers what it models: gradients computed in float64 but with the GPU
   path's roundings applied (dS and P rounded to bf16 before their products,
   D_i from a bf16-rounded O, the gradients rounded to bf16) stay within it,
   on inputs whose gradients are a small difference of large terms.
2. It is not vacuous: the gradients of a forward that counts a global key
   twice when it also lies in a row's band (the mistake the "dedup" inputs
   were made to expose; Longformer summary page, section 3-1 "Global
   Attention": every key once) leave it.
3. Its fp32 form (rounding 2^-20 per sum, plus the fp32 score and dP dot
   products) covers gradients computed entirely in float32.
"""
import numpy as np
import pytest
import torch

from oracle import allowed_mask, attention, attention_backward
from sliding_window_attention_banded_amd.workloads import Workload, make_inputs
from tests._bwd import FLOOR, GRADS, ROUND, SAFETY, cotangent, slice_bounds
from tests._lib import to64

WL = Workload("bound", 1, 2, 160, 64, (32, 16), (1, 2), False, (3, 40, 100))


def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).double().numpy()


def _rows_grads(Q, K, V, do, og, mask, s):
    """One kind of rows (regular or global) with the GPU path's roundings."""
    S = np.where(mask, s * (Q @ K.T), -np.inf)
    P = np.exp(S - S.max(axis=1, keepdims=True))
    P /= P.sum(axis=1, keepdims=True)
    dP = do @ V.T
    D = (do * og).sum(axis=1)                   # from the O the forward returned
    dS = _bf16(P * (dP - D[:, None]))
    return s * (dS @ K), s * (dS.T @ Q), _bf16(P).T @ do


def _simulated(t, do, og, wl, b, h, gl):
    n, d = t["q"].shape[2:]
    s = 1.0 / np.sqrt(d)
    rows = np.arange(n)
    mask = allowed_mask(rows, n, wl.window[h], wl.dilation[h], wl.causal, gl)
    isg = np.zeros(n, dtype=bool)
    isg[list(gl)] = True
    out = [np.zeros((n, d)) for _ in range(6)]
    for sel, names, base in ((~isg, ("q", "k", "v"), 0), (isg, ("qg", "kg", "vg"), 3)):
        Q, K, V = (t[x][b, h] for x in names)
        a, bk, bv = _rows_grads(Q[sel], K, V, do[b, h][sel], og[b, h][sel], mask[sel], s)
        out[base][sel] = a
        out[base + 1] += bk
        out[base + 2] += bv
    return [_bf16(x) for x in out]


def _double_counted(t, do, wl, b, h, gl):
    """Gradients (float64 autograd) of a forward in which a global key that
    also lies in a row's band enters that row's softmax twice."""
    n, d = t["q"].shape[2:]
    s = 1.0 / np.sqrt(d)
    T = {x: torch.from_numpy(t[x][b, h].copy()).requires_grad_(True) for x in t}
    rows = np.arange(n)
    mask = torch.from_numpy(allowed_mask(rows, n, wl.window[h], wl.dilation[h], wl.causal, gl))
    band = torch.from_numpy(allowed_mask(rows, n, wl.window[h], wl.dilation[h], wl.causal, []))
    g = torch.tensor(list(gl))
    isg = torch.zeros(n, dtype=torch.bool)
    isg[g] = True
    S = s * T["q"] @ T["k"].T
    S = torch.where(mask, S, torch.tensor(-np.inf, dtype=torch.float64))
    extra = torch.where(band[:, g], s * T["q"] @ T["k"][g].T, torch.tensor(-np.inf, dtype=torch.float64))
    P = torch.softmax(torch.cat([S, extra], dim=1), dim=1)
    O = P @ torch.cat([T["v"], T["v"][g]], dim=0)
    Sg = torch.where(mask, s * T["qg"] @ T["kg"].T, torch.tensor(-np.inf, dtype=torch.float64))
    Og = torch.softmax(Sg, dim=1) @ T["vg"]
    O = torch.where(isg[:, None], Og, O)
    (O * torch.from_numpy(do[b, h])).sum().backward()
    dq = torch.where(isg[:, None], torch.zeros(()), T["q"].grad)
    dqg = torch.where(isg[:, None], T["qg"].grad, torch.zeros(()))
    return [x.detach().numpy() for x in (dq, T["k"].grad, T["v"].grad, dqg, T["kg"].grad, T["vg"].grad)]


@pytest.mark.parametrize("kind", ["dedup", "sharp"])
def test_bound_covers_the_modelled_roundings(kind):
    inp = make_inputs(WL, 0, kind)
    dout = cotangent(WL, 0)
    t = {x: to64(inp[x]) for x in ("q", "k", "v", "qg", "kg", "vg")}
    do = to64(dout)
    o, _ = attention(t["q"], t["k"], t["v"], t["qg"], t["kg"], t["vg"], window=list(WL.window),
                     dilation=list(WL.dilation), causal=WL.causal, global_idx=list(WL.global_idx))
    og = _bf16(o)
    refs = attention_backward(t["q"], t["k"], t["v"], t["qg"], t["kg"], t["vg"], do,
                              window=list(WL.window), dilation=list(WL.dilation),
                              causal=WL.causal, global_idx=list(WL.global_idx))
    gl = list(WL.global_idx)
    worst = 0.0
    for h in range(WL.heads):
        bounds = slice_bounds(*(t[x][0, h] for x in ("q", "k", "v", "qg", "kg", "vg")), do[0, h],
                              og[0, h], WL.window[h], WL.dilation[h], WL.causal, gl)
        sim = _simulated(t, do, og, WL, 0, h, gl)
        for gi, name in enumerate(GRADS):
            r = refs[gi][0, h]
            bnd = SAFETY * (bounds[gi] + ROUND * np.abs(r)) + FLOOR
            ratio = float((np.abs(sim[gi] - r) / bnd).max())
            worst = max(worst, ratio)
            assert ratio <= 1.0, f"head {h} {name}: simulated error beyond the bound ({ratio:.3f})"
    # the modelled roundings use a fair share of the bound, not a vanishing one
    assert worst > 0.02


def test_bound_catches_a_double_counted_global_key():
    inp = make_inputs(WL, 0, "dedup")
    dout = cotangent(WL, 0)
    t = {x: to64(inp[x]) for x in ("q", "k", "v", "qg", "kg", "vg")}
    do = to64(dout)
    o, _ = attention(t["q"], t["k"], t["v"], t["qg"], t["kg"], t["vg"], window=list(WL.window),
                     dilation=list(WL.dilation), causal=WL.causal, global_idx=list(WL.global_idx))
    refs = attention_backward(t["q"], t["k"], t["v"], t["qg"], t["kg"], t["vg"], do,
                              window=list(WL.window), dilation=list(WL.dilation),
                              causal=WL.causal, global_idx=list(WL.global_idx))
    gl = list(WL.global_idx)
    caught = 0
    for h in range(WL.heads):
        bounds = slice_bounds(*(t[x][0, h] for x in ("q", "k", "v", "qg", "kg", "vg")), do[0, h],
                              _bf16(o)[0, h], WL.window[h], WL.dilation[h], WL.causal, gl)
        wrong = _double_counted(t, do, WL, 0, h, gl)
        for gi in (0, 1, 2):
            r = refs[gi][0, h]
            bnd = SAFETY * (bounds[gi] + ROUND * np.abs(r)) + FLOOR
            caught += int((np.abs(wrong[gi] - r) > bnd).any())
    assert caught >= 2


def _f32_grads(t, do, og, wl, h, gl):
    """Every gradient of one head computed in float32 from the float32 O."""
    f = np.float32
    n, d = t["q"].shape[2:]
    s = f(1.0 / np.sqrt(d))
    rows = np.arange(n)
    mask = allowed_mask(rows, n, wl.window[h], wl.dilation[h], wl.causal, gl)
    isg = np.zeros(n, dtype=bool)
    isg[list(gl)] = True
    out = [np.zeros((n, d), dtype=f) for _ in range(6)]
    for sel, names, base in ((~isg, ("q", "k", "v"), 0), (isg, ("qg", "kg", "vg"), 3)):
        Q, K, V = (t[x][0, h][sel if x[0] == "q" else slice(None)].astype(f) for x in names)
        dO, O = do[0, h][sel].astype(f), og[0, h][sel].astype(f)
        S = np.where(mask[sel], s * (Q @ K.T), f(-np.inf)).astype(f)
        m = S.max(axis=1, keepdims=True)
        P = np.exp(S - m).astype(f)
        P = (P / P.sum(axis=1, keepdims=True)).astype(f)
        dP = (dO @ V.T).astype(f)
        D = (dO * O).sum(axis=1, dtype=f)
        dS = (P * (dP - D[:, None])).astype(f)
        out[base][sel] = s * (dS @ K)
        out[base + 1] += s * (dS.T @ Q)
        out[base + 2] += P.T @ dO
    return [x.astype(np.float64) for x in out]


@pytest.mark.parametrize("kind", ["normal", "sharp", "dedup"])
def test_fp32_bound_covers_float32_gradients(kind):
    inp = make_inputs(WL, 1, kind)
    dout = cotangent(WL, 1)
    t = {x: to64(inp[x]) for x in ("q", "k", "v", "qg", "kg", "vg")}
    do = to64(dout)
    o, _ = attention(t["q"], t["k"], t["v"], t["qg"], t["kg"], t["vg"], window=list(WL.window),
                     dilation=list(WL.dilation), causal=WL.causal, global_idx=list(WL.global_idx))
    og = o.astype(np.float32).astype(np.float64)
    refs = attention_backward(t["q"], t["k"], t["v"], t["qg"], t["kg"], t["vg"], do,
                              window=list(WL.window), dilation=list(WL.dilation),
                              causal=WL.causal, global_idx=list(WL.global_idx))
    gl = list(WL.global_idx)
    worst = 0.0
    for h in range(WL.heads):
        bounds = slice_bounds(*(t[x][0, h] for x in ("q", "k", "v", "qg", "kg", "vg")), do[0, h],
                              og[0, h], WL.window[h], WL.dilation[h], WL.causal, gl,
                              rnd=2.0 ** -20, serr=2.0 ** -21)
        got = _f32_grads(t, do, og, WL, h, gl)
        for gi, name in enumerate(GRADS):
            r = refs[gi][0, h]
            bnd = SAFETY * (bounds[gi] + 2.0 ** -20 * np.abs(r)) + FLOOR
            ratio = float((np.abs(got[gi] - r) / bnd).max())
            worst = max(worst, ratio)
            assert ratio <= 1.0, f"head {h} {name}: float32 error beyond the fp32 bound ({ratio:.3f})"
    assert worst > 0.01
