"""Planted mistakes: each mutation of the oracle must fail a pin.

The mistakes are planted in the oracle itself (monkeypatched, on the CPU), and
the pins they must trip are the golden values derived by hand from the
Longformer summary page and the brute force of the page's definitions.
"""
import numpy as np
import pytest

import oracle.masked_softmax as oa
from tests.test_oracle_bruteforce import CASES, brute
from tests.test_oracle_golden import GOLD, _ln_case_inputs


def _golden_ok():
    for case in GOLD["ln_weights"]["cases"]:
        n = case["n"]
        o, lse = oa.attention(*_ln_case_inputs(n), window=case["window"],
                              dilation=case["dilation"], causal=case["causal"],
                              global_idx=case["global"])
        want = np.log(np.array(case["lse_of"], dtype=np.float64))
        if not np.allclose(lse[0, 0], want, rtol=0, atol=1e-12):
            return False
    return True


def _brute_ok(limit=300):
    rng = np.random.default_rng(0)
    for (n, w, dil, causal, G) in CASES[:limit]:
        t = [rng.standard_normal((1, 1, n, 3)) for _ in range(6)]
        o, _ = oa.attention(*t, window=w, dilation=dil, causal=causal,
                            global_idx=G)
        bo, _ = brute(*(x[0, 0].tolist() for x in t), w, dil, causal, G)
        if not np.allclose(o[0, 0], np.array(bo), rtol=0, atol=1e-12):
            return False
    return True


def test_unmutated_oracle_passes():
    assert _golden_ok() and _brute_ok()


def _wider_band(rows, n, window, dilation, causal):
    return _orig_band(rows, n, window + 2, dilation, causal)


def _undilated_band(rows, n, window, dilation, causal):
    return _orig_band(rows, n, window, 1, causal)


def _one_sided_band(rows, n, window, dilation, causal):
    m = _orig_band(rows, n, window, dilation, causal)
    i = np.asarray(rows)[:, None]
    return m & (np.arange(n)[None, :] >= i)


_orig_band = oa.band_mask


@pytest.mark.parametrize("mut", [_wider_band, _undilated_band,
                                 _one_sided_band])
def test_band_mutations_are_caught(monkeypatch, mut):
    monkeypatch.setattr(oa, "band_mask", mut)
    assert not (_golden_ok() and _brute_ok())


def test_wrong_scale_is_caught(monkeypatch):
    orig = oa._masked_softmax_rows
    monkeypatch.setattr(oa, "_masked_softmax_rows",
                        lambda qr, k, v, mask, scale: orig(qr, k, v, mask,
                                                           scale * scale))
    assert not _brute_ok()


def test_global_rows_with_regular_projections_are_caught(monkeypatch):
    orig = oa.attention

    def mutated(q, k, v, qg=None, kg=None, vg=None, **kw):
        return orig(q, k, v, q, k, v, **kw)
    monkeypatch.setattr(oa, "attention", mutated)
    assert not _golden_ok()


def test_missing_global_columns_are_caught(monkeypatch):
    orig = oa.allowed_mask

    def mutated(rows, n, window, dilation, causal, global_idx):
        m = orig(rows, n, window, dilation, causal, global_idx)
        g = np.zeros(n, bool)
        g[np.asarray(global_idx, dtype=np.int64)] = True
        band = _orig_band(rows, n, window, dilation, causal)
        reg = ~g[np.asarray(rows)]
        m[reg] = band[reg]
        return m
    monkeypatch.setattr(oa, "allowed_mask", mutated)
    assert not (_golden_ok() and _brute_ok())


def test_strict_causal_is_caught(monkeypatch):
    orig = oa.allowed_mask

    def mutated(rows, n, window, dilation, causal, global_idx):
        m = orig(rows, n, window, dilation, causal, global_idx)
        if causal:
            i = np.asarray(rows)[:, None]
            j = np.arange(n)[None, :]
            m &= (j < i) | (j == 0)
        return m
    monkeypatch.setattr(oa, "allowed_mask", mutated)
    assert not (_golden_ok() and _brute_ok())
