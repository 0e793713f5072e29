"""Pins of the oracle's backward pass (gradients of every input for a
cotangent dO of O), against what the mathematics fixes independently of it:

* the derivative that torch autograd takes through the library's scaled
  dot-product attention, on masks built here from the per-(i, j) predicates
  of the Longformer summary page (section 3-1; section 7 for causal);
* central finite differences of <dO, O> computed with the (pinned) forward
  oracle, on tiny inputs;
* closed forms: shifting every key by one vector leaves each row's softmax
  unchanged (so the dK rows sum to zero), the weights of a row sum to one (so
  the dV rows sum to the dO rows), rows of G take nothing from Q and rows
  off G nothing from Qg; and linearity in dO.

A planted mistake (the rowsum term of the softmax derivative dropped) must
fail the autograd pin.
"""
import numpy as np
import pytest
import torch

import oracle.masked_softmax as oa
from oracle import attention, attention_backward


def _allowed_ref(n, w, dil, causal, G):
    """[n, n] key sets written from the predicates, one (i, j) at a time."""
    Gs = set(G)
    m = np.zeros((n, n), dtype=bool)
    for i in range(n):
        for j in range(n):
            left_ok = (not causal) or j <= i
            if i in Gs:
                m[i, j] = left_ok
            else:
                in_band = abs(i - j) <= (w // 2) * dil and (i - j) % dil == 0
                m[i, j] = (in_band or j in Gs) and left_ok
    return m


def _autograd_ref(q, k, v, qg, kg, vg, do, w, dil, causal, G):
    """Gradients by torch autograd through scaled_dot_product_attention."""
    B, H, n, d = q.shape
    m = torch.from_numpy(_allowed_ref(n, w, dil, causal, G))
    isg = torch.zeros(n, dtype=torch.bool)
    isg[list(G)] = True
    ts = [torch.from_numpy(np.ascontiguousarray(x)).requires_grad_(True)
          for x in (q, k, v, qg, kg, vg)]
    o_reg = torch.nn.functional.scaled_dot_product_attention(ts[0], ts[1], ts[2], attn_mask=m)
    o_glb = torch.nn.functional.scaled_dot_product_attention(ts[3], ts[4], ts[5], attn_mask=m)
    o = torch.where(isg[None, None, :, None], o_glb, o_reg)
    (o * torch.from_numpy(do)).sum().backward()
    return [t.grad.numpy() for t in ts]


CASES = [
    # n, w, dil, causal, G
    (16, 4, 1, False, []),
    (16, 4, 1, True, []),
    (23, 6, 2, False, [0]),
    (23, 6, 3, True, [4, 11]),
    (40, 8, 1, False, [0, 1, 39]),
    (40, 10, 4, True, [7, 20, 33]),
    (33, 64, 1, False, [5]),       # window wider than the sequence
    (29, 0, 1, False, [3, 17]),    # window 0: a row sees itself and G
]


@pytest.mark.parametrize("n,w,dil,causal,G", CASES)
def test_backward_matches_autograd_through_sdpa(n, w, dil, causal, G):
    rng = np.random.default_rng(n * 7 + w)
    t = [rng.standard_normal((2, 2, n, 8)) for _ in range(7)]
    got = attention_backward(*t, window=w, dilation=dil, causal=causal, global_idx=G)
    want = _autograd_ref(*t, w, dil, causal, G)
    for name, a, b in zip(("dq", "dk", "dv", "dqg", "dkg", "dvg"), got, want):
        if a is None:  # no global tokens: the global projections take no part
            np.testing.assert_array_equal(b, 0.0)
            continue
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-11, err_msg=name)


def test_backward_row_blocks_do_not_change_the_result():
    rng = np.random.default_rng(3)
    t = [rng.standard_normal((1, 2, 50, 8)) for _ in range(7)]
    kw = dict(window=8, dilation=2, causal=True, global_idx=[3, 30])
    a = attention_backward(*t, **kw)
    b = attention_backward(*t, row_block=7, **kw)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_finite_differences(causal):
    rng = np.random.default_rng(11)
    n, d, w, dil, G = 9, 4, 4, 2, [2, 7]
    t = [rng.standard_normal((1, 1, n, d)) for _ in range(6)]
    do = rng.standard_normal((1, 1, n, d))
    kw = dict(window=w, dilation=dil, causal=causal, global_idx=G)

    def loss(xs):
        o, _ = attention(*xs, **kw)
        return float((o * do).sum())

    grads = attention_backward(*t, do, **kw)
    eps = 1e-6
    for which in range(6):
        u = rng.standard_normal(t[which].shape)
        xp = [x.copy() for x in t]
        xm = [x.copy() for x in t]
        xp[which] += eps * u
        xm[which] -= eps * u
        fd = (loss(xp) - loss(xm)) / (2 * eps)
        an = float((grads[which] * u).sum())
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (which, fd, an)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_closed_forms(causal):
    rng = np.random.default_rng(5)
    n, G = 60, [0, 13, 59]
    t = [rng.standard_normal((2, 3, n, 8)) for _ in range(7)]
    dq, dk, dv, dqg, dkg, dvg = attention_backward(
        *t, window=10, dilation=3, causal=causal, global_idx=G)
    do = t[6]
    isg = np.zeros(n, dtype=bool)
    isg[G] = True
    # a common shift of every key is a per-row constant on the scores
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)
    np.testing.assert_allclose(dkg.sum(axis=2), 0.0, atol=1e-12)
    # every row's weights sum to one
    np.testing.assert_allclose(dv.sum(axis=2), do[:, :, ~isg].sum(axis=2), atol=1e-12)
    np.testing.assert_allclose(dvg.sum(axis=2), do[:, :, isg].sum(axis=2), atol=1e-12)
    # rows of G use Qg only, the other rows Q only
    np.testing.assert_array_equal(dq[:, :, isg], 0.0)
    np.testing.assert_array_equal(dqg[:, :, ~isg], 0.0)


def test_backward_is_linear_in_do():
    rng = np.random.default_rng(8)
    t = [rng.standard_normal((1, 2, 30, 8)) for _ in range(6)]
    d1, d2 = rng.standard_normal((2, 1, 2, 30, 8))
    kw = dict(window=6, dilation=1, causal=False, global_idx=[4])
    g1 = attention_backward(*t, d1, **kw)
    g2 = attention_backward(*t, d2, **kw)
    g3 = attention_backward(*t, 2.0 * d1 - 0.5 * d2, **kw)
    for a, b, c in zip(g1, g2, g3):
        np.testing.assert_allclose(c, 2.0 * a - 0.5 * b, atol=1e-12)


def test_planted_missing_rowsum_term_fails(monkeypatch):
    def broken(qr, k, v, dor, mask, scale):
        s = np.where(mask, scale * (qr @ k.T), -np.inf)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        ds = p * (dor @ v.T)  # the -rowsum(P*dP) term dropped
        return scale * (ds @ k), scale * (ds.T @ qr), p.T @ dor

    monkeypatch.setattr(oa, "_masked_softmax_grad_rows", broken)
    n, w, dil, causal, G = CASES[3]
    rng = np.random.default_rng(n * 7 + w)
    t = [rng.standard_normal((2, 2, n, 8)) for _ in range(7)]
    got = oa.attention_backward(*t, window=w, dilation=dil, causal=causal, global_idx=G)
    want = _autograd_ref(*t, w, dil, causal, G)
    assert np.abs(got[0] - want[0]).max() > 1e-3
