"""Pins of the projection oracle (the step in front of the attention: the
Longformer summary page, section 3-1, "Linear Projections for Global
Attention"): the head/projection layout by block-identity weights, the bias
alone by zero weights, linearity, and the product against torch's
float64 linear layer on the same values.
"""
import numpy as np
import pytest
import torch

from oracle import project


def test_block_identity_weights_copy_the_input_into_the_head_layout():
    rng = np.random.default_rng(0)
    B, n, H = 2, 5, 3
    D = H * 64
    x = rng.standard_normal((B, n, D))
    w = np.concatenate([np.eye(D)] * 3, axis=0)  # q = k = v = x, head h = features 64h..
    for t in project(x, w, None, H):
        for h in range(H):
            np.testing.assert_array_equal(t[:, h], x[:, :, 64 * h:64 * h + 64])


def test_zero_weights_give_the_bias():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((1, 4, 128))
    bias = rng.standard_normal(6 * 2 * 64)
    outs = project(x, np.zeros((6 * 2 * 64, 128)), bias, 2)
    assert len(outs) == 6
    for p, t in enumerate(outs):
        for h in range(2):
            col = (p * 2 + h) * 64
            np.testing.assert_array_equal(t[0, h], np.broadcast_to(bias[col:col + 64], (4, 64)))


@pytest.mark.parametrize("P", [3, 6])
def test_matches_torch_linear(P):
    rng = np.random.default_rng(P)
    B, n, D, H = 2, 7, 192, 3
    x = rng.standard_normal((B, n, D))
    w = rng.standard_normal((P * H * 64, D))
    b = rng.standard_normal(P * H * 64)
    ref = torch.nn.functional.linear(torch.from_numpy(x), torch.from_numpy(w),
                                     torch.from_numpy(b)).numpy()  # [B, n, P*H*64]
    outs = project(x, w, b, H)
    for p in range(P):
        for h in range(H):
            c = (p * H + h) * 64
            np.testing.assert_allclose(outs[p][:, h], ref[:, :, c:c + 64], rtol=0, atol=1e-10)


def test_linear_in_x():
    rng = np.random.default_rng(4)
    x1, x2 = rng.standard_normal((2, 1, 3, 64))
    w = rng.standard_normal((3 * 64, 64))
    a = project(x1, w, None, 1)
    b = project(x2, w, None, 1)
    c = project(3.0 * x1 - x2, w, None, 1)
    for u, v, z in zip(a, b, c):
        np.testing.assert_allclose(z, 3.0 * u - v, atol=1e-12)


def test_rejects_bad_shapes():
    with pytest.raises(ValueError):
        project(np.zeros((1, 2, 64)), np.zeros((100, 64)), None, 1)


def test_planted_transposed_head_layout_fails():
    """Reading the output features as (head, projection) instead of
    (projection, head) must fail the torch pin above."""
    rng = np.random.default_rng(9)
    B, n, D, H, P = 1, 4, 64, 2, 3
    x = rng.standard_normal((B, n, D))
    w = rng.standard_normal((P * H * 64, D))
    ref = (x.reshape(n, D) @ w.T).reshape(n, P, H, 64)
    wrong = (x.reshape(n, D) @ w.T).reshape(n, H, P, 64).transpose(0, 2, 1, 3)
    outs = project(x, w, None, H)
    assert np.abs(wrong[:, 1, 0] - outs[1][0, 0]).max() > 1e-3
    np.testing.assert_allclose(ref[:, 1, 0], outs[1][0, 0], atol=1e-12)
