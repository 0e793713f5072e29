"""Float64 attention evaluated band by band, O(n * (w + R) * d).

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing on the product
path may import this module.

The same definition as ``masked_softmax.attention`` (Longformer summary page,
section 3-1 "Attention Pattern", section 7 for the left-only mask; readings
R1-R8 there), evaluated without the n x n mask:

* With dilation delta, row i only meets keys of its own residue class
  (i - j divisible by delta), and on that subsequence the dilated band is
  the plain band of w/2 keys on each side (w/2 to the left when causal). So
  each residue class is cut into blocks of R rows, and a block's scores are
  one product against the keys its rows can reach (its band span, R + w
  keys at most), masked to each row's own band.
* A row's global keys that are not already in its band (left of it when
  causal) are scored beside it; the softmax runs over both.
* A global row attends to every position (left of it when causal) with Qg,
  Kg, Vg, as in the dense form.

This is the CPU cost of the method's own key sets (band blocks instead of
n x n), a second evaluation of the definition, and the banded CPU reference
of the benchmark.
"""

from __future__ import annotations

import numpy as np

from .masked_softmax import _per_batch_globals

__all__ = ["attention_banded"]


def _softmax_rows(s):
    """Row softmax of scores with -inf outside the key set, and its LSE."""
    mx = s.max(axis=1, keepdims=True)
    p = np.exp(s - mx)
    den = p.sum(axis=1, keepdims=True)
    return p / den, mx[:, 0] + np.log(den[:, 0])


def attention_banded(q, k, v, qg=None, kg=None, vg=None, *, window, dilation,
                     causal=False, global_idx=(), row_block=128):
    """O [B,H,n,d] and LSE [B,H,n] in float64 (all rows).

    Arguments as ``masked_softmax.attention``; ``row_block`` is R, the rows
    of one residue class scored together.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, n, d = q.shape
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one [B,H,n,d] shape")
    gls = _per_batch_globals(global_idx, B, n)
    if any(gl.size for gl in gls):
        qg = np.asarray(qg, dtype=np.float64)
        kg = np.asarray(kg, dtype=np.float64)
        vg = np.asarray(vg, dtype=np.float64)
    win = np.broadcast_to(np.asarray(window, dtype=np.int64), (H,))
    dil = np.broadcast_to(np.asarray(dilation, dtype=np.int64), (H,))
    if (win < 0).any() or (win % 2).any() or (dil < 1).any():
        raise ValueError("windows must be even and >= 0, dilations >= 1")
    scale = 1.0 / np.sqrt(d)

    o = np.zeros((B, H, n, d), dtype=np.float64)
    lse = np.zeros((B, H, n), dtype=np.float64)
    for b in range(B):
        gl = np.sort(gls[b])
        isg = np.zeros(n, dtype=bool)
        isg[gl] = True
        for h in range(H):
            half, delta = int(win[h]) // 2, int(dil[h])
            right = 0 if causal else half
            kh, vh = k[b, h], v[b, h]
            for r in range(min(delta, n)):
                pos = np.arange(r, n, delta, dtype=np.int64)      # residue class r
                nr = pos.size
                for t0 in range(0, nr, row_block):
                    t = np.arange(t0, min(nr, t0 + row_block), dtype=np.int64)
                    t = t[~isg[pos[t]]]                          # non-global rows
                    if t.size == 0:
                        continue
                    u0 = max(0, int(t[0]) - half)
                    u1 = min(nr, int(t[-1]) + right + 1)
                    u = np.arange(u0, u1, dtype=np.int64)        # the block's key span
                    off = u[None, :] - t[:, None]
                    qi = q[b, h, pos[t]]
                    sb = scale * (qi @ kh[pos[u]].T)
                    sb = np.where((off >= -half) & (off <= right), sb, -np.inf)
                    if gl.size:
                        diff = pos[t][:, None] - gl[None, :]
                        inband = ((diff % delta) == 0) & (diff <= half * delta) & (diff >= -right * delta)
                        keep = ~inband & ((diff >= 0) if causal else True)
                        sg = np.where(keep, scale * (qi @ kh[gl].T), -np.inf)
                        p, ll = _softmax_rows(np.concatenate([sb, sg], axis=1))
                        o[b, h, pos[t]] = p[:, :u.size] @ vh[pos[u]] + p[:, u.size:] @ vh[gl]
                    else:
                        p, ll = _softmax_rows(sb)
                        o[b, h, pos[t]] = p @ vh[pos[u]]
                    lse[b, h, pos[t]] = ll
            for g in gl:                                           # global rows
                top = g + 1 if causal else n
                s = scale * (kg[b, h, :top] @ qg[b, h, g])
                mx = s.max()
                p = np.exp(s - mx)
                o[b, h, g] = (p @ vg[b, h, :top]) / p.sum()
                lse[b, h, g] = mx + np.log(p.sum())
    return o, lse
