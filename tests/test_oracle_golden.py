"""Oracle against values derived by hand from the page's definitions.

The fixture tests/golden/hand_derived.json holds, for tiny cases, the key set
of every row and the exact output and log-sum-exp, worked out by hand from the
Longformer summary page, section 3-1 (sliding window, dilated window, global
attention, separate global projections) and section 7 (left-only mask).
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import allowed_mask, attention

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                   "hand_derived.json")))


def _ln_case_inputs(n):
    q = np.ones((1, 1, n, 1))
    k = np.log(np.arange(1, n + 1, dtype=np.float64)).reshape(1, 1, n, 1)
    v = np.arange(n, dtype=np.float64).reshape(1, 1, n, 1)
    qg = np.ones((1, 1, n, 1))
    kg = np.log(n - np.arange(n, dtype=np.float64)).reshape(1, 1, n, 1)
    vg = 2.0 * np.arange(n, dtype=np.float64).reshape(1, 1, n, 1)
    return q, k, v, qg, kg, vg


@pytest.mark.parametrize("case", GOLD["ln_weights"]["cases"],
                         ids=lambda c: c["name"])
def test_ln_weight_cases(case):
    n = case["n"]
    q, k, v, qg, kg, vg = _ln_case_inputs(n)
    o, lse = attention(q, k, v, qg, kg, vg, window=case["window"],
                       dilation=case["dilation"], causal=case["causal"],
                       global_idx=case["global"])
    want_o = np.array([float(Fraction(x)) for x in case["o"]])
    want_lse = np.log(np.array(case["lse_of"], dtype=np.float64))
    np.testing.assert_allclose(o[0, 0, :, 0], want_o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse[0, 0], want_lse, rtol=0, atol=1e-13)
    m = allowed_mask(np.arange(n), n, case["window"], case["dilation"],
                     case["causal"], case["global"])
    for i, keys in enumerate(case["keys"]):
        assert sorted(np.nonzero(m[i])[0].tolist()) == keys, i


@pytest.mark.parametrize("case", GOLD["uniform_sets"]["cases"],
                         ids=lambda c: c["name"])
def test_uniform_sets(case):
    n = case["n"]
    z = np.zeros((1, 1, n, n))
    eye = np.eye(n).reshape(1, 1, n, n)
    o, lse = attention(z, z, eye, z, z, eye, window=case["window"],
                       dilation=case["dilation"], causal=case["causal"],
                       global_idx=case["global"])
    for i, keys in enumerate(case["keys"]):
        want = np.zeros(n)
        want[keys] = 1.0 / len(keys)
        np.testing.assert_allclose(o[0, 0, i], want, rtol=0, atol=1e-15)
        assert abs(lse[0, 0, i] - math.log(len(keys))) < 1e-14
