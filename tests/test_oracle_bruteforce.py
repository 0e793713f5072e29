"""Pin P1: the vectorised oracle against a per-(i, j) brute force.

The brute force enumerates each row's keys the way the Longformer summary page
describes them (section 3-1): w/2 keys on each side spaced by the dilation,
every global token, and for a global row every token with the separate global
projections; the left-only mask of section 7 drops keys to the right. It uses
pure Python and math.exp, and shares nothing with the oracle's predicates.
"""
import itertools
import math
import random

import numpy as np
import pytest

from oracle import attention


def brute(q, k, v, qg, kg, vg, window, dilation, causal, G):
    n, d = len(q), len(q[0])
    s = 1.0 / math.sqrt(d)
    Gs = set(G)
    out, lses = [], []
    for i in range(n):
        if i in Gs:
            keys = [j for j in range(n) if (not causal or j <= i)]
            qq, kk, vv = qg, kg, vg
        else:
            keys = set()
            for t in range(-(window // 2), window // 2 + 1):
                j = i + t * dilation
                if 0 <= j < n:
                    keys.add(j)
            keys |= Gs
            keys = sorted(j for j in keys if (not causal or j <= i))
            qq, kk, vv = q, k, v
        sc = [s * sum(qq[i][c] * kk[j][c] for c in range(d)) for j in keys]
        mx = max(sc)
        ws = [math.exp(x - mx) for x in sc]
        tot = sum(ws)
        out.append([sum(w * vv[j][c] for w, j in zip(ws, keys)) / tot
                    for c in range(d)])
        lses.append(mx + math.log(tot))
    return out, lses


def _grid():
    rng = random.Random(1234)
    cases = []
    for n in (1, 2, 5, 7, 12):
        gsets = [(), (0,), (n - 1,), tuple(sorted(rng.sample(range(n), min(n, 3))))]
        for w in range(0, 2 * n + 4, 2):
            for dil in (1, 2, 3, 5):
                for causal in (False, True):
                    for G in gsets:
                        cases.append((n, w, dil, causal, tuple(sorted(set(G)))))
    return sorted(set(cases))


CASES = _grid()


@pytest.mark.parametrize("chunk", range(8))
def test_oracle_matches_bruteforce(chunk):
    rng = np.random.default_rng(chunk)
    d = 3
    for (n, w, dil, causal, G) in CASES[chunk::8]:
        q, k, v, qg, kg, vg = (rng.standard_normal((1, 1, n, d)) for _ in range(6))
        o, lse = attention(q, k, v, qg, kg, vg, window=w, dilation=dil,
                           causal=causal, global_idx=G)
        bo, bl = brute(q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist(),
                       qg[0, 0].tolist(), kg[0, 0].tolist(), vg[0, 0].tolist(),
                       w, dil, causal, G)
        np.testing.assert_allclose(o[0, 0], np.array(bo), rtol=0, atol=1e-12,
                                   err_msg=str((n, w, dil, causal, G)))
        np.testing.assert_allclose(lse[0, 0], np.array(bl), rtol=0, atol=1e-12)


def test_grid_is_exhaustive_enough():
    # every (dilation, causal) pair meets windows beyond 2n and empty/edge G
    assert len(CASES) > 1000
    combos = {(c[2], c[3], c[1] >= 2 * c[0]) for c in CASES}
    assert len(combos) == 16
