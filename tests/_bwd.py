"""Backward-pass test helpers: the cotangent, the GPU run, and a per-element
error bound for the gradients derived from the arithmetic of the GPU path.

Why a per-element bound: a gradient element can be a small difference of
large terms (dq_i = s sum_j dS_ij k_j with dS_ij = P_ij (dO_i.v_j - D_i), and
D_i = dO_i.O_i), so a bound relative to the result, or to the tensor's
largest element, cannot hold where the terms cancel. The bound below sums
the magnitudes of the terms instead.

Rounding the GPU path performs (bf16 inputs, fp32 accumulation):
  * dS (and P, for dV) enter their MFMAs rounded to bf16: relative 2^-9 each
    (round to nearest even, 8 significant bits); taken as 2^-8 to cover the
    fp32 sums of up to ~2*10^4 products (n * 2^-24 < 2^-9 there);
  * D_i is formed from the O that the forward returned in bf16, not from the
    exact O: |delta D_i| = |dO_i . (O_gpu,i - O_i)| plus fp32 rounding;
  * every gradient is rounded to bf16 at the end: relative 2^-8 (with margin).
First-order propagation gives, per element (d is the feature index):
  |d dq_id| <= s (2^-8 sum_j |dS_ij| |k_jd| + |delta D_i| sum_j P_ij |k_jd|) + 2^-8 |dq_id|
  |d dk_jd| <= s (2^-8 sum_i |dS_ij| |q_id| + sum_i P_ij |delta D_i| |q_id|)  + 2^-8 |dk_jd|
  |d dv_jd| <= 2^-8 sum_i P_ij |dO_id| + 2^-8 |dv_jd|
and the same for the global rows with Qg, Kg, Vg. Tests allow twice that,
plus 1e-6 absolute for elements whose exact value is 0.

P, dS and D come from float64 evaluations of the oracle's own key sets
(oracle.allowed_mask), one (batch, head) slice and block of rows at a time.
"""
import numpy as np
import torch

from sliding_window_attention_banded_amd.workloads import item_globals

GRADS = ("dq", "dk", "dv", "dqg", "dkg", "dvg")
ROUND = 2.0 ** -8
SAFETY = 2.0
FLOOR = 1e-6


def cotangent(wl, seed):
    g = torch.Generator().manual_seed(10_000 + seed)
    return torch.randn((wl.batch, wl.heads, wl.n, wl.d), generator=g).to(wl.torch_dtype)


def gpu_forward_backward(wl, inp, dout):
    """(O, LSE, gradients) of the HIP library, on the CPU."""
    from sliding_window_attention_banded_amd import Plan
    dev = {k: (v.cuda() if v is not None else None) for k, v in inp.items()}
    with Plan(wl.batch, wl.heads, wl.n, wl.d, wl.window, wl.dilation, wl.causal,
              wl.global_idx, wl.torch_dtype) as pl:
        o, lse = pl.forward(dev["q"], dev["k"], dev["v"], dev["qg"], dev["kg"], dev["vg"],
                            want_lse=True)
        grads = pl.backward(dev["q"], dev["k"], dev["v"], o, lse, dout.cuda(),
                            dev["qg"], dev["kg"], dev["vg"])
        torch.cuda.synchronize()
    return o.cpu(), lse.cpu(), [None if t is None else t.cpu() for t in grads]


def slice_bounds(q, k, v, qg, kg, vg, do, og, window, dilation, causal, gl, row_block=1024,
                 rnd=ROUND, serr=0.0):
    """The sums of term magnitudes above for one (batch, head): [n, d]
    float64 arrays in, (bq, bk, bv, bqg, bkg, bvg) out (the last three None
    without global tokens); the final-rounding term is added by the caller.

    ``serr`` > 0 adds the rounding of the fp32 dot products themselves, which
    the bf16 path's 2^-8 terms dwarf but the fp32 path does not: a score
    q.k summed in fp32 is off by up to serr * sum_d |q_d k_d|, so P_ij is off
    by P_ij (s * that + serr) (the exponential and the LSE add about one
    more unit), and dP_ij = dO_i.v_j by serr * sum_d |dO_d v_d|; then
    |d dS_ij| <= (dP error) P_ij + (P error) |dP_ij - D_i|,
    and these enter dq, dk as |dS| does and dv through P."""
    from oracle import allowed_mask
    n, d = q.shape
    s = 1.0 / np.sqrt(d)
    gl = np.asarray(gl, dtype=np.int64)
    isg = np.zeros(n, dtype=bool)
    isg[gl] = True
    out = [np.zeros((n, d)) for _ in range(3)]
    outg = [np.zeros((n, d)) for _ in range(3)] if gl.size else [None] * 3
    for s0 in range(0, n, row_block):
        rb = np.arange(s0, min(n, s0 + row_block))
        mask = allowed_mask(rb, n, window, dilation, causal, gl)
        for sel, (Q, K, V), (BQ, BK, BV) in ((~isg[rb], (q, k, v), out),
                                             (isg[rb], (qg, kg, vg), outg)):
            if not sel.any():
                continue
            r = rb[sel]
            S = s * (Q[r] @ K.T)
            S = np.where(mask[sel], S, -np.inf)
            P = np.exp(S - S.max(axis=1, keepdims=True))
            P /= P.sum(axis=1, keepdims=True)
            O = P @ V
            dP = do[r] @ V.T
            D = (P * dP).sum(axis=1)
            adS = np.abs(P * (dP - D[:, None]))
            dD = np.abs(((og[r] - O) * do[r]).sum(axis=1)) + \
                2.0 ** -22 * (np.abs(og[r]) * np.abs(do[r])).sum(axis=1)
            aK, aQ, adO = np.abs(K), np.abs(Q[r]), np.abs(do[r])
            BQ[r] = s * (rnd * (adS @ aK) + dD[:, None] * (P @ aK))
            BK += s * (rnd * (adS.T @ aQ) + (P * dD[:, None]).T @ aQ)
            BV += rnd * (P.T @ adO)
            if serr:
                dPr = P * (s * serr * (aQ @ aK.T) + serr)       # |error of P|
                edS = dPr * np.abs(dP - D[:, None]) + P * serr * (adO @ np.abs(V).T)
                BQ[r] += s * (edS @ aK)
                BK += s * (edS.T @ aQ)
                BV += dPr.T @ adO
    return tuple(out) + tuple(outg)


def check_grads(wl, inp, dout, o_gpu, got, refs, bh=None, label="", rel=1e-2, rnd=ROUND,
                serr=0.0):
    """Every gradient element within SAFETY * (its bound + the final
    rounding of the reference) + FLOOR; with ``rel``, also the relative RMS
    of each tensor (a global sanity check for inputs without cancellation).
    ``bh`` restricts the check to (batch, head) slices; ``refs`` then holds
    one tuple of six slice gradients per slice, else the six full tensors.
    ``rnd`` is the relative rounding of the path's arithmetic (2^-8 for the
    bf16 path; for fp32, a few units of 2^-24 per sum); ``serr`` that of the
    fp32 dot products (see slice_bounds)."""
    f = lambda t: None if t is None else t.double().numpy()
    t = {k: f(inp[k]) for k in ("q", "k", "v", "qg", "kg", "vg")}
    do, og = f(dout), f(o_gpu)
    slices = bh if bh is not None else [(b, h) for b in range(wl.batch) for h in range(wl.heads)]
    gls = item_globals(wl)
    worst = 0.0
    for idx, (b, h) in enumerate(slices):
        sl = lambda x: None if x is None else x[b, h]
        bounds = slice_bounds(sl(t["q"]), sl(t["k"]), sl(t["v"]), sl(t["qg"]), sl(t["kg"]),
                              sl(t["vg"]), do[b, h], og[b, h], wl.window[h], wl.dilation[h],
                              wl.causal, list(gls[b]), rnd=rnd, serr=serr)
        for gi, name in enumerate(GRADS):
            r = refs[idx][gi] if bh is not None else refs[gi]
            if r is None:
                assert got[gi] is None, f"{label}: {name} should be absent"
                continue
            rr = r[0, 0] if bh is not None else r[b, h]
            g = got[gi][b, h].double().numpy()
            assert np.isfinite(g).all(), f"{label}[{b},{h}]: non-finite {name}"
            # an item without global tokens has no terms in its global gradients
            terms = bounds[gi] if bounds[gi] is not None else 0.0
            bnd = SAFETY * (terms + rnd * np.abs(rr)) + FLOOR
            err = np.abs(g - rr)
            ratio = float((err / bnd).max())
            worst = max(worst, ratio)
            if ratio > 1.0:
                where = np.unravel_index((err / bnd).argmax(), err.shape)
                raise AssertionError(f"{label}[{b},{h}]/{name}: error {err[where]:.3e} above its "
                                     f"bound {bnd[where]:.3e} at {where}")
    if rel is not None:
        for gi, name in enumerate(GRADS):
            if got[gi] is None:
                continue
            if bh is None:
                g, r = got[gi].double().numpy(), refs[gi]
            else:
                g = np.stack([got[gi][b, h].double().numpy() for b, h in slices])
                r = np.stack([refs[i][gi][0, 0] for i in range(len(slices))])
            rms = np.sqrt((r ** 2).mean())
            if rms > FLOOR:
                e = np.sqrt(((g - r) ** 2).mean()) / rms
                assert e <= rel, f"{label}/{name}: rel-rms {e:.3e}"
    print(f"  {label}: worst error / bound {worst:.3f}", flush=True)
    return worst
