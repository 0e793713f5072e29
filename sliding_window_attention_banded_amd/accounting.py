"""Algorithmic work and traffic of one forward pass, from closed forms.

Used by the benchmark to turn a measured time into TFLOP/s and GB/s. Nothing
here runs on the device and nothing here is on the compute path.

Key counts follow the pattern of the Longformer summary page, section 3-1: a
row i keeps w/2 keys on each side, spaced by the head's dilation, clipped at
the sequence ends; with the left-only mask the right side is empty. Written
as a closed form per row:

    |band(i)| = min(floor(i / delta), w/2)
              + [not causal] * min(floor((n - 1 - i) / delta), w/2) + 1
"""

from __future__ import annotations

import numpy as np

__all__ = ["band_keys_per_row", "band_flops", "useful_flops",
           "algorithmic_bytes", "global_column_extras", "backward_flops", "backward_bytes"]


def band_keys_per_row(n, window, dilation, causal):
    """Closed-form |band(i)| for i = 0..n-1 (int64 array)."""
    i = np.arange(n, dtype=np.int64)
    half = window // 2
    left = np.minimum(i // dilation, half)
    right = 0 if causal else np.minimum((n - 1 - i) // dilation, half)
    return left + right + 1


def band_flops(wl):
    """4*d*sum of |band(i)| over every (batch, head, row): QK^T plus PV."""
    tot = 0
    for h in range(wl.heads):
        tot += int(band_keys_per_row(wl.n, wl.window[h], wl.dilation[h],
                                     wl.causal).sum())
    return 4 * wl.d * wl.batch * tot


def global_column_extras(n, window, dilation, causal, global_idx):
    """Per row: number of global keys outside the row's band (and left of it
    when causal); rows that are themselves global get 0."""
    g = np.asarray(sorted(global_idx), dtype=np.int64)
    i = np.arange(n, dtype=np.int64)
    if g.size == 0:
        return np.zeros(n, dtype=np.int64)
    diff = i[:, None] - g[None, :]
    half = window // 2
    inband = (np.abs(diff) <= half * dilation) & (diff % dilation == 0)
    if causal:
        inband &= diff >= 0
        ok = diff >= 0
    else:
        ok = np.ones_like(inband)
    extra = (ok & ~inband).sum(axis=1)
    extra[g] = 0
    return extra


def useful_flops(wl):
    """4*d*(keys actually attended): band keys of non-global rows, plus the
    global columns outside their bands, plus every key of each global row
    (per batch item, with that item's global set)."""
    from .workloads import item_globals
    sets = item_globals(wl)
    tot = 0
    for gs in set(sets):
        mult = sets.count(gs)
        g = np.asarray(gs, dtype=np.int64)
        for h in range(wl.heads):
            kb = band_keys_per_row(wl.n, wl.window[h], wl.dilation[h], wl.causal)
            ex = global_column_extras(wl.n, wl.window[h], wl.dilation[h], wl.causal, gs)
            keep = np.ones(wl.n, dtype=bool)
            keep[g] = False
            t = int(kb[keep].sum() + ex.sum())
            if g.size:
                t += int((g + 1).sum()) if wl.causal else int(g.size * wl.n)
            tot += mult * t
    return 4 * wl.d * tot


def algorithmic_bytes(wl, with_lse=True):
    """Bytes that must cross HBM once: Q, K, V read and O written; with
    global tokens also Kg, Vg in full and the Qg rows; plus the fp32 LSE."""
    from .workloads import item_globals
    es = 2 if wl.dtype == "bf16" else 4
    bh = wl.batch * wl.heads
    b = 4 * bh * wl.n * wl.d * es
    for gs in item_globals(wl):  # Kg, Vg of items with global tokens, and their Qg rows
        if gs:
            b += wl.heads * (2 * wl.n + len(gs)) * wl.d * es
    if with_lse:
        b += 4 * bh * wl.n
    return b


def backward_flops(wl):
    """Algorithmic FLOPs of the backward pass: five products per attended
    (row, key) pair -- the recomputed scores q.k, dP = dO.v, and the three
    gradient products dq += dS k, dk += dS q, dv += P dO -- at 2*d each,
    i.e. 2.5 times the forward's 4*d per pair."""
    return useful_flops(wl) * 10 // 4


def backward_bytes(wl):
    """Bytes that must cross HBM once in the backward pass: Q, K, V, O, dO and
    the LSE read, dQ, dK, dV written; with global tokens also Kg, Vg read in
    full with the Qg rows, and dQg, dKg, dVg written in full."""
    from .workloads import item_globals
    es = 2 if wl.dtype == "bf16" else 4
    bh = wl.batch * wl.heads
    row = wl.d * es
    b = bh * wl.n * (5 * row + 4 + 3 * row)
    for gs in item_globals(wl):
        if gs:
            b += wl.heads * (wl.n * (2 * row + 3 * row) + len(gs) * row)
    return b
