"""Randomised GPU parity: configurations drawn from a fixed seed (batch,
heads, ragged n, per-head windows and dilations including window 0, windows
wider than the sequence and dilations beyond it, causal or not, no / shared /
per-item global tokens), each run through the forward and the backward and
compared with the float64 oracle element by element, with the tolerances of
tests/test_gpu_parity.py (forward) and tests/_bwd.py (backward: a bound per
element from the magnitudes of the terms it sums, which also holds where the
"dedup" inputs make a gradient a small difference of large terms). The draw
is part of the test, so every run checks the same configurations."""
import numpy as np
import pytest
import torch

from sliding_window_attention_banded_amd.workloads import Workload, item_globals, make_inputs
from tests._lib import compare, ensure_library, oracle_ref, to64

pytestmark = pytest.mark.gpu

N_CONFIGS = 64


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_library()


def _draw(i):
    rng = np.random.default_rng(1000 + i)
    B = int(rng.integers(1, 4))
    H = int(rng.integers(1, 5))
    n = int(rng.integers(1, 40)) if rng.random() < 0.2 else int(rng.integers(40, 700))

    def one_window():
        u = rng.random()
        if u < 0.1:
            return 0
        if u < 0.35:
            return int(2 * rng.integers(0, 3 * n // 2 + 2))  # up to beyond the sequence
        return int(2 * rng.integers(1, 65))
    win = tuple(one_window() for _ in range(H))
    dil = tuple(int(rng.integers(1, 5)) if rng.random() < 0.8 else int(rng.integers(1, n + 2))
                for _ in range(H))
    causal = i % 3 == 0
    mode = (i // 3) % 3  # none / shared / per item, crossed with causal
    if mode == 0:
        G = ()
    elif mode == 1:
        k = int(rng.integers(1, min(n, 80) + 1))
        G = tuple(sorted(int(x) for x in rng.choice(n, size=k, replace=False)))
    else:
        sets = []
        for _ in range(B):
            k = int(rng.integers(0, min(n, 80) + 1))
            sets.append(tuple(int(x) for x in rng.choice(n, size=k, replace=False)))
        G = tuple(sets)
    kind = ("normal", "sharp", "dedup")[int(rng.integers(0, 3))]
    return Workload(f"rand{i}", B, H, n, 64, win, dil, causal, G, "bf16"), kind


def _draw_one_global(i):
    """At most one global token per batch item (the configuration in which
    the band blocks fold the global column in from registers): a shared
    token, or one per item with some items having none."""
    wl, kind = _draw(2000 + i)
    rng = np.random.default_rng(3000 + i)
    n, B = wl.n, wl.batch
    if i % 2 == 0:
        G = (int(rng.integers(0, n)),)
    else:
        G = tuple(((int(rng.integers(0, n)),) if rng.random() < 0.7 else ()) for _ in range(B))
    return Workload(f"rand1g{i}", B, wl.heads, n, 64, wl.window, wl.dilation, i % 4 < 2, G,
                    "bf16"), kind


CONFIGS = [_draw(i) for i in range(N_CONFIGS)] + [_draw_one_global(i) for i in range(16)]


@pytest.mark.parametrize("wl,kind", CONFIGS, ids=[c[0].name for c in CONFIGS])
def test_random_config_forward_and_backward(wl, kind):
    from oracle import attention_backward
    from tests._bwd import check_grads, cotangent
    print(f"[rand] {wl.name} B{wl.batch} H{wl.heads} n{wl.n} win={wl.window} dil={wl.dilation} "
          f"causal={wl.causal} G-sizes={[len(s) for s in item_globals(wl)]} kind={kind}", flush=True)
    inp = make_inputs(wl, 7, kind)
    dout = cotangent(wl, 7)
    ref_o, ref_lse = oracle_ref(wl, inp)
    o, lse = _run_gpu(wl, inp)
    compare(wl, o, lse, ref_o, ref_lse, label=wl.name)
    grads = _run_gpu(wl, inp, dout)
    t = [to64(inp[k]) for k in ("q", "k", "v", "qg", "kg", "vg")] + [to64(dout)]
    refs = attention_backward(*t, window=list(wl.window), dilation=list(wl.dilation),
                              causal=wl.causal, global_idx=list(wl.global_idx))
    check_grads(wl, inp, dout, o, grads, refs, label=wl.name,
                rel=None if kind == "dedup" else 1e-2)


def _run_gpu(wl, inp, dout=None):
    """O and LSE on the GPU, or with a cotangent the backward's gradients."""
    from sliding_window_attention_banded_amd import Plan
    dev = {k: (v.cuda() if v is not None else None) for k, v in inp.items()}
    with Plan(wl.batch, wl.heads, wl.n, 64, wl.window, wl.dilation, wl.causal,
              wl.global_idx, torch.bfloat16) as pl:
        o, lse = pl.forward(dev["q"], dev["k"], dev["v"], dev["qg"], dev["kg"], dev["vg"],
                            want_lse=True)
        if dout is None:
            torch.cuda.synchronize()
            return o.cpu(), lse.cpu()
        grads = pl.backward(dev["q"], dev["k"], dev["v"], o, lse, dout.cuda(),
                            dev["qg"], dev["kg"], dev["vg"])
        torch.cuda.synchronize()
    return [None if g is None else g.cpu() for g in grads]
