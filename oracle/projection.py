"""Float64 oracle of the projection step in front of the attention.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The Longformer summary page (section 3-1, "Linear Projections for Global
Attention") computes the attention's queries, keys and values with linear
projections of the layer input, and uses a second, separate set of
projections Qg, Kg, Vg for global attention. For input rows x (one per token,
d_model features) and head h, projection p of head h is

    P[b, h, i, e] = sum_c x[b, i, c] * W[(p * H + h) * 64 + e, c]
                    + bias[(p * H + h) * 64 + e]

with W stored one output feature per row (the layout of a linear layer's
weight, out_features x in_features) and the projections in the order q, k, v
(then qg, kg, vg when global tokens are used). The scale 1/sqrt(64) is not
folded in (the attention applies it).
"""

from __future__ import annotations

import numpy as np

__all__ = ["project"]


def project(x, w, bias, heads):
    """x [B, n, D], w [P*heads*64, D], bias [P*heads*64] or None ->
    list of P arrays [B, heads, n, 64], float64."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    B, n, D = x.shape
    if w.ndim != 2 or w.shape[1] != D or w.shape[0] % (heads * 64) or w.shape[0] == 0:
        raise ValueError("w must be [P*heads*64, d_model]")
    P = w.shape[0] // (heads * 64)
    y = x.reshape(B * n, D) @ w.T
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)[None, :]
    y = y.reshape(B, n, P, heads, 64)
    return [np.ascontiguousarray(y[:, :, p].transpose(0, 2, 1, 3)) for p in range(P)]
