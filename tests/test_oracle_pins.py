"""Pins P2-P12: the oracle against closed forms, library reductions and
invariants that the Longformer summary page (section 3-1, section 7) and the
mathematics of softmax fix.
"""
import numpy as np
import pytest
import torch

from oracle import allowed_mask, attention, band_mask
from sliding_window_attention_banded_amd.accounting import (
    band_keys_per_row, global_column_extras)


def _rand(rng, B, H, n, d, k=6):
    return [rng.standard_normal((B, H, n, d)) for _ in range(k)]


# ---- P2: closed-form key counts equal the mask row sums -------------------
@pytest.mark.parametrize("n", [1, 3, 17, 64, 129])
@pytest.mark.parametrize("w", [0, 2, 8, 64, 300])
@pytest.mark.parametrize("dil", [1, 2, 3, 4])
@pytest.mark.parametrize("causal", [False, True])
def test_p2_key_counts(n, w, dil, causal):
    m = band_mask(np.arange(n), n, w, dil, causal)
    np.testing.assert_array_equal(m.sum(1), band_keys_per_row(n, w, dil, causal))


@pytest.mark.parametrize("causal", [False, True])
def test_p2_global_extras(causal):
    n, w, dil = 200, 16, 3
    G = [0, 5, 60, 61, 150, 199]
    full = allowed_mask(np.arange(n), n, w, dil, causal, G)
    band = band_mask(np.arange(n), n, w, dil, causal)
    extra = (full & ~band).sum(1)
    extra[G] = 0
    np.testing.assert_array_equal(extra, global_column_extras(n, w, dil, causal, G))


# ---- P3: textbook reduction to scaled dot-product attention ----------------
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,d", [(1, 4), (33, 8), (100, 64)])
def test_p3_full_window_is_sdpa(causal, n, d):
    rng = np.random.default_rng(n)
    q, k, v = _rand(rng, 2, 3, n, d, 3)
    o, lse = attention(q, k, v, window=2 * n + (2 * n) % 2, dilation=1,
                       causal=causal)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        is_causal=causal).numpy()
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)
    s = np.einsum("bhid,bhjd->bhij", q, k) / np.sqrt(d)
    if causal:
        s = np.where(np.tril(np.ones((n, n), bool)), s, -np.inf)
    np.testing.assert_allclose(lse, np.logaddexp.reduce(s, axis=-1), atol=1e-12)


def test_p3_window_just_short_of_full_differs():
    rng = np.random.default_rng(0)
    n = 20
    q, k, v = _rand(rng, 1, 1, n, 8, 3)
    o, _ = attention(q, k, v, window=2 * (n - 2), dilation=1)
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(t) for t in (q, k, v))).numpy()
    # rows 0 and n-1 lose one key each; the rest still see everything
    assert np.abs(o - ref)[0, 0, [0, n - 1]].max() > 1e-3
    np.testing.assert_allclose(o[0, 0, 1:-1], ref[0, 0, 1:-1], atol=1e-12)


# ---- P4: global rows are full attention with the global projections --------
@pytest.mark.parametrize("causal", [False, True])
def test_p4_global_rows_are_full_attention(causal):
    rng = np.random.default_rng(4)
    n, d = 90, 16
    q, k, v, qg, kg, vg = _rand(rng, 2, 2, n, d)
    G = [0, 7, 44, 89]
    o, _ = attention(q, k, v, qg, kg, vg, window=6, dilation=2, causal=causal,
                     global_idx=G)
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(t) for t in (qg, kg, vg)), is_causal=causal).numpy()
    np.testing.assert_allclose(o[:, :, G], ref[:, :, G], rtol=0, atol=1e-12)


# ---- P5: convexity and exact support ---------------------------------------
@pytest.mark.parametrize("causal", [False, True])
def test_p5_constant_values(causal):
    rng = np.random.default_rng(5)
    n, d = 70, 8
    q, k, _, qg, kg, _ = _rand(rng, 1, 2, n, d)
    c = rng.standard_normal(d)
    v = np.broadcast_to(c, (1, 2, n, d))
    o, _ = attention(q, k, v, qg, kg, v, window=10, dilation=3, causal=causal,
                     global_idx=[3, 50])
    np.testing.assert_allclose(o, np.broadcast_to(c, o.shape), atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dil", [1, 2, 5])
def test_p5_identity_values_expose_the_support(causal, dil):
    rng = np.random.default_rng(dil)
    n = 24
    q, k, _, qg, kg, _ = _rand(rng, 1, 1, n, n)
    eye = np.eye(n).reshape(1, 1, n, n)
    G = [2, 13]
    o, _ = attention(q, k, eye, qg, kg, eye, window=4, dilation=dil,
                     causal=causal, global_idx=G)
    P = o[0, 0]
    A = allowed_mask(np.arange(n), n, 4, dil, causal, G)
    assert (P[A] > 0).all() and (P[~A] == 0).all()
    np.testing.assert_allclose(P.sum(1), 1.0, atol=1e-14)


# ---- P6: zero queries give the plain mean over the key set -----------------
def test_p6_uniform_scores_mean():
    rng = np.random.default_rng(6)
    n, d = 57, 5
    _, k, v, _, kg, vg = _rand(rng, 1, 1, n, d)
    z = np.zeros((1, 1, n, d))
    G = [0, 30]
    o, lse = attention(z, k, v, z, kg, vg, window=8, dilation=2, causal=False,
                       global_idx=G)
    A = allowed_mask(np.arange(n), n, 8, 2, False, G)
    for i in range(n):
        src = vg if i in G else v
        np.testing.assert_allclose(o[0, 0, i], src[0, 0, A[i]].mean(0), atol=1e-14)
        assert abs(lse[0, 0, i] - np.log(A[i].sum())) < 1e-14


# ---- P7: dilation is the undilated window on residue subsequences ----------
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dil,n", [(2, 64), (3, 50), (4, 23)])
def test_p7_dilation_is_residue_subsequences(causal, dil, n):
    rng = np.random.default_rng(dil * 10 + n)
    q, k, v = _rand(rng, 1, 1, n, 8, 3)
    w = 6
    o, lse = attention(q, k, v, window=w, dilation=dil, causal=causal)
    for r in range(dil):
        sl = slice(r, None, dil)
        o2, l2 = attention(q[:, :, sl], k[:, :, sl], v[:, :, sl], window=w,
                           dilation=1, causal=causal)
        np.testing.assert_allclose(o[:, :, sl], o2, atol=1e-13)
        np.testing.assert_allclose(lse[:, :, sl], l2, atol=1e-13)


# ---- P8: separation of the two projection sets -----------------------------
def test_p8_projection_separation():
    rng = np.random.default_rng(8)
    n, d = 80, 8
    q, k, v, qg, kg, vg = _rand(rng, 1, 2, n, d)
    G = [1, 40, 79]
    kw = dict(window=10, dilation=1, causal=False, global_idx=G)
    o, _ = attention(q, k, v, qg, kg, vg, **kw)
    reg = np.setdiff1d(np.arange(n), G)
    # perturbing the global projections leaves regular rows unchanged
    o2, _ = attention(q, k, v, qg + 1.0, kg * 2.0, vg - 3.0, **kw)
    np.testing.assert_array_equal(o[:, :, reg], o2[:, :, reg])
    assert np.abs(o[:, :, G] - o2[:, :, G]).max() > 0.1
    # perturbing regular projections at regular positions leaves global rows
    q3, k3, v3 = q.copy(), k.copy(), v.copy()
    q3[:, :, reg] += 1.0
    k3[:, :, reg] *= 2.0
    v3[:, :, reg] -= 3.0
    o3, _ = attention(q3, k3, v3, qg, kg, vg, **kw)
    np.testing.assert_array_equal(o[:, :, G], o3[:, :, G])


# ---- P9: LSE-merge identity --------------------------------------------------
@pytest.mark.parametrize("causal", [False, True])
def test_p9_lse_merge_of_band_and_globals(causal):
    rng = np.random.default_rng(9)
    n, d, w, dil = 120, 8, 16, 2
    q, k, v, qg, kg, vg = _rand(rng, 1, 1, n, d)
    G = [0, 3, 64, 65, 119]
    o, lse = attention(q, k, v, qg, kg, vg, window=w, dilation=dil,
                       causal=causal, global_idx=G)
    ob, lb = attention(q, k, v, window=w, dilation=dil, causal=causal)
    band = band_mask(np.arange(n), n, w, dil, causal)
    s = (q[0, 0] @ k[0, 0].T) / np.sqrt(d)
    for i in np.setdiff1d(np.arange(n), G):
        extra = [g for g in G if not band[i, g] and (not causal or g <= i)]
        if not extra:
            np.testing.assert_allclose(o[0, 0, i], ob[0, 0, i], atol=1e-14)
            continue
        se = s[i, extra]
        lg = np.logaddexp.reduce(se)
        og = (np.exp(se - lg)[:, None] * v[0, 0, extra]).sum(0)
        L = np.logaddexp(lb[0, 0, i], lg)
        merged = np.exp(lb[0, 0, i] - L) * ob[0, 0, i] + np.exp(lg - L) * og
        np.testing.assert_allclose(o[0, 0, i], merged, atol=1e-13)
        assert abs(lse[0, 0, i] - L) < 1e-13


# ---- P10: symmetry of the non-causal band --------------------------------
@pytest.mark.parametrize("w,dil", [(0, 1), (6, 1), (6, 3), (40, 2)])
def test_p10_symmetric_mask(w, dil):
    n = 61
    m = allowed_mask(np.arange(n), n, w, dil, False, [])
    np.testing.assert_array_equal(m, m.T)
    assert m.diagonal().all()


# ---- P11: receptive field grows by w/2 * dilation per layer --------------
@pytest.mark.parametrize("w,dil", [(2, 1), (4, 1), (4, 3), (8, 2)])
def test_p11_receptive_field(w, dil):
    n = 200
    m = band_mask(np.arange(n), n, w, dil, False).astype(np.int64)
    reach = np.eye(n, dtype=np.int64)
    centre = n // 2
    for layers in range(1, 5):
        reach = np.minimum(reach @ m, 1)
        cols = np.nonzero(reach[centre])[0]
        assert cols.max() - centre == layers * (w // 2) * dil
        assert centre - cols.min() == layers * (w // 2) * dil
        # dilation keeps the key count of a single layer at w + 1
    assert m[centre].sum() == w + 1


# ---- P12: linearity in V, invariance to a per-row score shift --------------
def test_p12_linearity_and_shift():
    rng = np.random.default_rng(12)
    n, d = 48, 6
    q, k, v1, _, _, v2 = _rand(rng, 1, 1, n, d)
    kw = dict(window=8, dilation=1, causal=True)
    o1, _ = attention(q, k, v1, **kw)
    o2, _ = attention(q, k, v2, **kw)
    o12, _ = attention(q, k, 2.0 * v1 - 0.5 * v2, **kw)
    np.testing.assert_allclose(o12, 2.0 * o1 - 0.5 * o2, atol=1e-13)
    # append a coordinate: q gets c_i * sqrt(d+1), k gets 1 -> every score of
    # row i moves by c_i; the output must not move and the LSE moves by c_i
    c = rng.standard_normal(n)
    qa = np.concatenate([q * np.sqrt((d + 1) / d), (c * np.sqrt(d + 1))[None, None, :, None]], -1)
    ka = np.concatenate([k, np.ones((1, 1, n, 1))], -1)
    va = np.concatenate([v1, np.zeros((1, 1, n, 1))], -1)
    oa, la = attention(qa, ka, va, **kw)
    ob, lb = attention(q, k, v1, **kw)
    np.testing.assert_allclose(oa[..., :d], ob, atol=1e-12)
    np.testing.assert_allclose(la - lb, c[None, None, :], atol=1e-12)


def test_rows_subset_matches_full():
    rng = np.random.default_rng(13)
    n, d = 300, 8
    q, k, v, qg, kg, vg = _rand(rng, 2, 2, n, d)
    kw = dict(window=[10, 20], dilation=[1, 3], causal=False, global_idx=[0, 9])
    o, lse = attention(q, k, v, qg, kg, vg, **kw)
    rows = [0, 1, 9, 150, 299]
    o2, l2 = attention(q, k, v, qg, kg, vg, rows=rows, row_block=2, **kw)
    np.testing.assert_allclose(o[:, :, rows], o2, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse[:, :, rows], l2, rtol=0, atol=1e-14)


def test_rejects_bad_arguments():
    z = np.zeros((1, 1, 4, 2))
    with pytest.raises(ValueError):
        attention(z, z, z, window=3, dilation=1)
    with pytest.raises(ValueError):
        attention(z, z, z, window=2, dilation=0)
    with pytest.raises(ValueError):
        attention(z, z, z, z, z, z, window=2, dilation=1, global_idx=[1, 1])
    with pytest.raises(ValueError):
        attention(z, z, z, z, z, z, window=2, dilation=1, global_idx=[4])
