"""Test helpers: build-if-missing for the HIP library, GPU runs and parity."""
import os
import re

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "swattn.h")


def ensure_library():
    from sliding_window_attention_banded_amd import binding, build
    if not os.path.exists(binding.library_path()):
        build.build()
    return binding.load_library()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(swattn_\w+)\s*\(",
                                 text, re.M)))


def to64(t):
    return None if t is None else t.double().numpy()


def run_gpu(wl, inp, want_lse=True, plan=None):
    from sliding_window_attention_banded_amd import Plan
    pl = plan or Plan(wl.batch, wl.heads, wl.n, wl.d, wl.window, wl.dilation,
                      wl.causal, wl.global_idx, wl.torch_dtype)
    dev = {k: (v.cuda() if v is not None else None) for k, v in inp.items()}
    o, lse = pl.forward(dev["q"], dev["k"], dev["v"], dev["qg"], dev["kg"],
                        dev["vg"], want_lse=want_lse)
    torch.cuda.synchronize()
    if plan is None:
        pl.close()
    return o.cpu(), (lse.cpu() if lse is not None else None)


def oracle_ref(wl, inp, rows=None):
    from oracle import attention
    return attention(to64(inp["q"]), to64(inp["k"]), to64(inp["v"]),
                     to64(inp["qg"]), to64(inp["kg"]), to64(inp["vg"]),
                     window=list(wl.window), dilation=list(wl.dilation),
                     causal=wl.causal, global_idx=list(wl.global_idx), rows=rows)


# Tolerances. bf16 I/O with fp32 accumulation: max-abs 2e-2 on O, plus a
# relative RMS bound. The row sum adds the unrounded fp32 weights (only the
# P V product takes them rounded to bf16), so the LSE carries fp32 rounding
# of the scores, the exponentials and a sum of at most a few thousand terms:
# far below the 1e-3 bound. fp32 path: 1e-5 on O and LSE.
TOL = {"bf16": dict(o=2e-2, rel=1e-2, lse=1e-3),
       "fp32": dict(o=1e-5, rel=2e-6, lse=1e-5)}


def compare(wl, o, lse, ref_o, ref_lse, rows=None, label=""):
    tol = TOL[wl.dtype]
    got = o.double().numpy()
    if rows is not None:
        got = got[:, :, rows]
    err = np.abs(got - ref_o)
    assert np.isfinite(got).all(), f"{label}: non-finite output"
    rel = np.sqrt((err ** 2).mean()) / max(np.sqrt((ref_o ** 2).mean()), 1e-30)
    where = np.unravel_index(err.argmax(), err.shape)
    assert err.max() <= tol["o"], f"{label}: max-abs {err.max():.3e} at {where}"
    assert rel <= tol["rel"], f"{label}: rel-rms {rel:.3e}"
    if lse is not None:
        gl = lse.double().numpy()
        if rows is not None:
            gl = gl[:, :, rows]
        lerr = np.abs(gl - ref_lse).max()
        assert lerr <= tol["lse"], f"{label}: lse max-abs {lerr:.3e}"
    return float(err.max()), float(rel)
