"""Explicit n x n masked-softmax attention in float64 (the oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing on the product
path may import this module.

What is computed, for one (batch, head) with window ``w`` and dilation ``delta``
(Longformer summary page, section 3-1):

* band(i, j)  <=>  |i - j| <= (w/2) * delta  and  (i - j) mod delta == 0.
  "Sliding Window": a token attends to w/2 tokens on each side.
  "Dilated Sliding Window": the window keeps its size (its number of keys)
  while gaps of ``delta`` widen the span it covers.
* caus(i, j)  <=>  not causal  or  j <= i
  (section 7: the decoder's self-attention looks left only).
* A non-global row i attends to  A(i) = {j : (band(i, j) or j in G) and
  caus(i, j)}  with the regular Q, K, V ("Global Attention": every token
  attends to the global tokens; a global key already in the band counts once).
* A global row g attends to every j with caus(g, j), using the separate global
  projections Qg, Kg, Vg ("Linear Projections for Global Attention").
* O_i = sum_{j in A(i)} softmax_j(s * q_i . k_j) v_j  with s = 1/sqrt(d), and
  LSE_i = ln sum_{j in A(i)} exp(s * q_i . k_j).

Readings taken where the page is silent or garbled:

* R1  the window is +-w/2 keys inclusive, so an interior row has w+1 keys;
      w must be even.
* R2  dilation puts keys at i +- k*delta for k <= w/2 (span w*delta, key count
      unchanged), which is what "keeps the compute, widens the receptive
      field" means; the printed O(n*w*d) contradicts the same sentence.
* R3  causal keeps the same band on the left: keys i - k*delta, 0 <= k <= w/2.
* R4  the softmax scale is 1/sqrt(d) (the page writes no formula).
* R5  global rows use Qg, Kg, Vg over all positions; global columns use the
      regular K[G], V[G], so each row is one softmax over one projection set.
* R6  a global key inside a row's band counts once (set union).
* R7  causal applies to global rows and columns too.
* R8  G is shared by every head; dilation applies to the band only. G is one
      set for all batch items, or one set per batch item (the QA setting of
      section 3-1: each example's question tokens are its global tokens);
      ``global_idx`` then lists B sequences.
"""

from __future__ import annotations

import numpy as np

__all__ = ["band_mask", "global_row_mask", "allowed_mask", "attention", "attention_backward"]


def band_mask(rows, n, window, dilation, causal):
    """Boolean [len(rows), n]: band(i, j) and caus(i, j) for i in ``rows``.

    Section 3-1 "Sliding Window" / "Dilated Sliding Window" (readings R1-R3).
    """
    if window < 0 or window % 2:
        raise ValueError("window must be even and >= 0")
    if dilation < 1:
        raise ValueError("dilation must be >= 1")
    i = np.asarray(rows, dtype=np.int64)[:, None]
    j = np.arange(n, dtype=np.int64)[None, :]
    diff = i - j
    m = (np.abs(diff) <= (window // 2) * dilation) & (diff % dilation == 0)
    if causal:
        m &= j <= i
    return m


def global_row_mask(rows, n, causal):
    """Boolean [len(rows), n] for global rows: every key, left only if causal.

    Section 3-1 "Global Attention" (a global token attends to all tokens), R7.
    """
    i = np.asarray(rows, dtype=np.int64)[:, None]
    j = np.arange(n, dtype=np.int64)[None, :]
    m = np.ones((i.shape[0], n), dtype=bool)
    if causal:
        m &= j <= i
    return m


def allowed_mask(rows, n, window, dilation, causal, global_idx):
    """Boolean [len(rows), n]: the key set A(i) of every row in ``rows``.

    Non-global rows: (band or j in G) and caus (R5-R7). Global rows: every
    key allowed by caus. Section 3-1, all four bullets.
    """
    rows = np.asarray(rows, dtype=np.int64)
    g = np.zeros(n, dtype=bool)
    g[np.asarray(global_idx, dtype=np.int64)] = True
    m = band_mask(rows, n, window, dilation, False)
    m |= g[None, :]
    if causal:
        m &= np.arange(n)[None, :] <= rows[:, None]
    rg = g[rows]
    if rg.any():
        m[rg] = global_row_mask(rows[rg], n, causal)
    return m


def _masked_softmax_rows(qr, k, v, mask, scale):
    """softmax(scale * qr k^T restricted to mask) v, and its log-sum-exp.

    Plain definition of attention over an explicit key set: scores, -inf
    outside the set, subtract the row max, exponentiate, normalise, multiply.
    """
    s = scale * (qr @ k.T)
    s = np.where(mask, s, -np.inf)
    mx = s.max(axis=1, keepdims=True)
    p = np.exp(s - mx)
    den = p.sum(axis=1, keepdims=True)
    o = (p @ v) / den
    lse = mx[:, 0] + np.log(den[:, 0])
    return o, lse


def _per_batch_globals(global_idx, B, n):
    """G of every batch item: a flat sequence (shared) or B sequences."""
    items = list(global_idx) if not isinstance(global_idx, np.ndarray) else list(global_idx.reshape(-1))
    per = bool(items) and all(isinstance(x, (list, tuple, np.ndarray)) for x in items)
    if per:
        if len(items) != B:
            raise ValueError("per-example global_idx needs one sequence per batch item")
        gls = [np.asarray(x, dtype=np.int64).reshape(-1) for x in items]
    else:
        gls = [np.asarray(items, dtype=np.int64).reshape(-1)] * B
    for gl in gls:
        if gl.size:
            if len(np.unique(gl)) != gl.size:
                raise ValueError("global_idx repeats an index")
            if gl.min() < 0 or gl.max() >= n:
                raise ValueError("global_idx out of range")
    return gls


def attention(q, k, v, qg=None, kg=None, vg=None, *, window, dilation,
              causal=False, global_idx=(), rows=None, row_block=1024):
    """Oracle forward: O [B,H,R,d] and LSE [B,H,R] in float64.

    ``q, k, v`` (and ``qg, kg, vg`` when G is not empty) are [B,H,n,d] arrays;
    they are upcast to float64 exactly. ``window`` and ``dilation`` are per
    head (sequences of length H) or scalars. ``rows`` selects which rows to
    compute (default: all n); R = len(rows). ``global_idx`` (one set for
    every batch item, or B sets: reading R8) may be unsorted but must not
    repeat.

    Each row block builds the explicit [rows x n] mask and evaluates the
    masked softmax directly (section 3-1; readings R1-R8 above).
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
        for t in (qg, kg, vg):
            if t.shape != q.shape:
                raise ValueError("qg, kg, vg must have q's shape")
    win = np.broadcast_to(np.asarray(window, dtype=np.int64), (H,))
    dil = np.broadcast_to(np.asarray(dilation, dtype=np.int64), (H,))
    rows = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    scale = 1.0 / np.sqrt(d)

    R = rows.size
    o = np.zeros((B, H, R, d), dtype=np.float64)
    lse = np.zeros((B, H, R), dtype=np.float64)
    for b in range(B):
        gl = gls[b]
        isg = np.zeros(n, dtype=bool)
        isg[gl] = True
        for h in range(H):
            for s0 in range(0, R, row_block):
                rb = rows[s0:s0 + row_block]
                mask = allowed_mask(rb, n, int(win[h]), int(dil[h]), causal, gl)
                reg = ~isg[rb]
                if reg.any():
                    oo, ll = _masked_softmax_rows(q[b, h, rb[reg]], k[b, h],
                                                  v[b, h], mask[reg], scale)
                    o[b, h, s0 + np.nonzero(reg)[0]] = oo
                    lse[b, h, s0 + np.nonzero(reg)[0]] = ll
                if (~reg).any():
                    oo, ll = _masked_softmax_rows(qg[b, h, rb[~reg]], kg[b, h],
                                                  vg[b, h], mask[~reg], scale)
                    o[b, h, s0 + np.nonzero(~reg)[0]] = oo
                    lse[b, h, s0 + np.nonzero(~reg)[0]] = ll
    return o, lse


def _masked_softmax_grad_rows(qr, k, v, dor, mask, scale):
    """Gradients of O = softmax(scale * qr k^T restricted to mask) v for the
    cotangent ``dor``: returns (dqr, dk, dv) with dk, dv over all n keys.

    The chain rule written out from the definition of the softmax: with P the
    row-normalised weights, dV = P^T dO, dP = dO V^T, dS = P * (dP - rowsum(P
    * dP)), dQ = scale * dS K, dK = scale * dS^T Q.
    """
    s = scale * (qr @ k.T)
    s = np.where(mask, s, -np.inf)
    mx = s.max(axis=1, keepdims=True)
    p = np.exp(s - mx)
    p /= p.sum(axis=1, keepdims=True)
    dp = dor @ v.T
    ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    return scale * (ds @ k), scale * (ds.T @ qr), p.T @ dor


def attention_backward(q, k, v, qg, kg, vg, do, *, window, dilation, causal=False,
                       global_idx=(), row_block=1024):
    """Oracle backward: gradients of every input for the cotangent ``do`` of O.

    Returns (dq, dk, dv, dqg, dkg, dvg), float64 arrays of q's shape; the
    global-projection gradients are None when G is empty (for every batch
    item). ``global_idx`` is one set or B sets, as in ``attention``. A non-global row i
    depends on q_i and on k_j, v_j for j in A(i); a global row g on qg_g and
    on kg_j, vg_j for every allowed j (section 3-1, readings R1-R8). Rows of G
    take their output from the global projections only, so dq is zero there,
    and dqg is zero off G.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, H, n, d = q.shape
    for t in (k, v, do):
        if t.shape != q.shape:
            raise ValueError("k, v, do must have q's [B,H,n,d] shape")
    gls = _per_batch_globals(global_idx, B, n)
    anyg = any(gl.size for gl in gls)
    if anyg:
        qg = np.asarray(qg, dtype=np.float64)
        kg = np.asarray(kg, dtype=np.float64)
        vg = np.asarray(vg, dtype=np.float64)
        for t in (qg, kg, vg):
            if t.shape != q.shape:
                raise ValueError("qg, kg, vg must have q's shape")
    win = np.broadcast_to(np.asarray(window, dtype=np.int64), (H,))
    dil = np.broadcast_to(np.asarray(dilation, dtype=np.int64), (H,))
    scale = 1.0 / np.sqrt(d)

    dq, dk, dv = np.zeros_like(q), np.zeros_like(q), np.zeros_like(q)
    if anyg:
        dqg, dkg, dvg = np.zeros_like(q), np.zeros_like(q), np.zeros_like(q)
    else:
        dqg = dkg = dvg = None
    rows = np.arange(n)
    for b in range(B):
        gl = gls[b]
        isg = np.zeros(n, dtype=bool)
        isg[gl] = True
        for h in range(H):
            for s0 in range(0, n, row_block):
                rb = rows[s0:s0 + row_block]
                mask = allowed_mask(rb, n, int(win[h]), int(dil[h]), causal, gl)
                reg = ~isg[rb]
                if reg.any():
                    r = rb[reg]
                    a, bk, bv = _masked_softmax_grad_rows(q[b, h, r], k[b, h], v[b, h],
                                                          do[b, h, r], mask[reg], scale)
                    dq[b, h, r] = a
                    dk[b, h] += bk
                    dv[b, h] += bv
                if (~reg).any():
                    r = rb[~reg]
                    a, bk, bv = _masked_softmax_grad_rows(qg[b, h, r], kg[b, h], vg[b, h],
                                                          do[b, h, r], mask[~reg], scale)
                    dqg[b, h, r] = a
                    dkg[b, h] += bk
                    dvg[b, h] += bv
    return dq, dk, dv, dqg, dkg, dvg
