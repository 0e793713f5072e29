"""Pins of per-example global tokens (one G per batch item: the QA setting of
the Longformer summary page, section 3-1 "Global Attention", where each
example's question tokens are its global tokens).

Each batch item is its own problem, so the oracle with B sets of global
tokens must equal, item by item, the per-(i, j) brute force (pure Python)
with that item's set, and the oracle run on that item alone with a shared
set; the backward likewise. A planted mistake (every item given item 0's
set) must fail.
"""
import numpy as np
import pytest

import oracle.masked_softmax as om
from oracle import attention, attention_backward
from tests.test_oracle_bruteforce import brute

SETS = [
    # n, window, dilation, causal, per-item G
    (9, 4, 1, False, [[0], [3, 8], [], [1, 2, 4]]),
    (11, 2, 2, True, [[5], [0, 10], [7], []]),
    (12, 6, 3, False, [[], [], [11], [0, 6]]),
]


@pytest.mark.parametrize("n,w,dil,causal,Gs", SETS)
def test_per_example_matches_brute_force(n, w, dil, causal, Gs):
    rng = np.random.default_rng(n + w)
    B = len(Gs)
    t = [rng.standard_normal((B, 1, n, 3)) for _ in range(6)]
    o, lse = attention(*t, window=w, dilation=dil, causal=causal, global_idx=Gs)
    for b in range(B):
        bo, bl = brute(*(x[b, 0].tolist() for x in t), w, dil, causal, Gs[b])
        np.testing.assert_allclose(o[b, 0], np.array(bo), rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[b, 0], np.array(bl), rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_per_example_is_itemwise_shared(causal):
    rng = np.random.default_rng(7)
    B, H, n = 3, 2, 80
    Gs = [[0, 40], [], [5, 6, 7, 79]]
    t = [rng.standard_normal((B, H, n, 8)) for _ in range(7)]
    kw = dict(window=[8, 12], dilation=[1, 3], causal=causal)
    o, lse = attention(*t[:6], global_idx=Gs, **kw)
    grads = attention_backward(*t, global_idx=Gs, **kw)
    for b in range(B):
        sl = [x[b:b + 1] for x in t]
        ob, lb = attention(*sl[:6], global_idx=Gs[b], **kw)
        np.testing.assert_array_equal(o[b:b + 1], ob)
        np.testing.assert_array_equal(lse[b:b + 1], lb)
        gb = attention_backward(*sl, global_idx=Gs[b], **kw)
        for a, c in zip(grads[:3], gb[:3]):
            np.testing.assert_array_equal(a[b:b + 1], c)
        for a, c in zip(grads[3:], gb[3:]):
            if c is None:  # this item has no global tokens
                np.testing.assert_array_equal(a[b:b + 1], 0.0)
            else:
                np.testing.assert_array_equal(a[b:b + 1], c)


def test_per_example_rejects_bad_sets():
    t = [np.zeros((2, 1, 5, 2)) for _ in range(6)]
    with pytest.raises(ValueError):
        attention(*t, window=2, dilation=1, global_idx=[[0]])        # one set for two items
    with pytest.raises(ValueError):
        attention(*t, window=2, dilation=1, global_idx=[[0, 0], []])  # repeat
    with pytest.raises(ValueError):
        attention(*t, window=2, dilation=1, global_idx=[[5], []])     # out of range


def test_planted_first_items_set_for_all_fails(monkeypatch):
    orig = om._per_batch_globals

    def broken(global_idx, B, n):
        gls = orig(global_idx, B, n)
        return [gls[0]] * B

    monkeypatch.setattr(om, "_per_batch_globals", broken)
    n, w, dil, causal, Gs = SETS[0]
    rng = np.random.default_rng(n + w)
    B = len(Gs)
    t = [rng.standard_normal((B, 1, n, 3)) for _ in range(6)]
    o, _ = om.attention(*t, window=w, dilation=dil, causal=causal, global_idx=Gs)
    worst = max(np.abs(o[b, 0] - np.array(brute(*(x[b, 0].tolist() for x in t), w, dil,
                                                 causal, Gs[b])[0])).max() for b in range(B))
    assert worst > 1e-3
