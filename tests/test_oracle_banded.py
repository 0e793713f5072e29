"""Pins of the key-enumerating oracle (``oracle.attention_banded``).

It evaluates the definition of the Longformer summary page (section 3-1;
section 7 for the left-only mask) over each row's enumerated keys instead of
an n x n mask. It is pinned against the per-(i, j) brute force of
``test_oracle_bruteforce`` on every tiny case of that grid, and against the
dense oracle (itself pinned) on seeded random shapes: per-head windows and
dilations, causal, shared and per-item global sets, windows wider than the
sequence and dilations beyond it. A planted mistake (the band one key too
narrow) must fail the comparison.
"""
import numpy as np
import pytest

from oracle import attention, attention_banded
from tests.test_oracle_bruteforce import CASES, brute


def _inputs(rng, B, H, n, d, with_g):
    t = lambda: rng.standard_normal((B, H, n, d)) * 1.5
    q, k, v = t(), t(), t()
    qg, kg, vg = (t(), t(), t()) if with_g else (None, None, None)
    return q, k, v, qg, kg, vg


@pytest.mark.parametrize("case", CASES[::7], ids=lambda c: f"n{c[0]}_w{c[1]}_d{c[2]}_c{int(c[3])}_G{len(c[4])}")
def test_banded_equals_brute_force(case):
    n, w, dil, causal, G = case
    rng = np.random.default_rng(n * 1000 + w * 10 + dil)
    q, k, v, qg, kg, vg = _inputs(rng, 1, 1, n, 3, True)
    o, lse = attention_banded(q, k, v, qg, kg, vg, window=w, dilation=dil, causal=causal,
                              global_idx=G)
    bo, bl = brute(q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist(), qg[0, 0].tolist(),
                   kg[0, 0].tolist(), vg[0, 0].tolist(), w, dil, causal, G)
    assert np.abs(o[0, 0] - np.array(bo)).max() < 1e-12
    assert np.abs(lse[0, 0] - np.array(bl)).max() < 1e-12


def _random_case(i):
    rng = np.random.default_rng(7000 + i)
    B, H = int(rng.integers(1, 4)), int(rng.integers(1, 4))
    n = int(rng.integers(1, 300))
    win = [2 * int(rng.integers(0, 3 * n // 2 + 2)) for _ in range(H)]
    dil = [int(rng.choice([1, 1, 2, 3, 7, n + 1])) for _ in range(H)]
    causal = bool(rng.random() < 0.5)
    kind = rng.integers(0, 3)
    if kind == 0:
        G = ()
    elif kind == 1:
        G = tuple(sorted(rng.choice(n, size=min(n, int(rng.integers(1, 6))), replace=False).tolist()))
    else:
        G = tuple(tuple(sorted(rng.choice(n, size=min(n, int(rng.integers(0, 6))), replace=False).tolist()))
                  for _ in range(B))
    return B, H, n, win, dil, causal, G


@pytest.mark.parametrize("i", range(40))
def test_banded_equals_dense_oracle(i):
    B, H, n, win, dil, causal, G = _random_case(i)
    rng = np.random.default_rng(i)
    q, k, v, qg, kg, vg = _inputs(rng, B, H, n, 8, True)
    o, lse = attention_banded(q, k, v, qg, kg, vg, window=win, dilation=dil, causal=causal,
                              global_idx=G, row_block=37)
    ro, rl = attention(q, k, v, qg, kg, vg, window=win, dilation=dil, causal=causal,
                       global_idx=G)
    assert np.abs(o - ro).max() < 1e-12
    assert np.abs(lse - rl).max() < 1e-12


def test_planted_narrow_band_fails():
    """The band one key narrower on each side must not pass for the true
    definition (the comparison can see a wrong window)."""
    rng = np.random.default_rng(3)
    q, k, v, qg, kg, vg = _inputs(rng, 1, 2, 90, 8, True)
    o, _ = attention_banded(q, k, v, qg, kg, vg, window=[10, 6], dilation=[1, 2], global_idx=(4,))
    wrong, _ = attention(q, k, v, qg, kg, vg, window=[8, 4], dilation=[1, 2], global_idx=(4,))
    assert np.abs(o - wrong).max() > 1e-3
