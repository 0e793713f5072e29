"""GPU parity of the projections in front of the attention (the separate
local and global Q/K/V projections of the Longformer summary page, section
3-1, "Linear Projections for Global Attention"): the HIP library's
swattn_project against the float64 oracle, element by element, on the same
bf16 inputs.

Tolerance, from the arithmetic: the products of two bf16 values are exact in
fp32; the fp32 accumulation of D of them (and the bias) is off by at most
about (D+1) * 2^-24 * A, A = sum_c |x_c w_c| + |bias| (the MFMA's own
summation order is not IEEE left-to-right, so the test allows 4x that: E);
the result is then rounded once to bf16 (relative 2^-8 at most). So
|got - ref| <= 2^-8 * (|ref| + E) + E per element, and the relative RMS
error, dominated by the final rounding, stays under 2^-8.
"""
import numpy as np
import pytest
import torch

from sliding_window_attention_banded_amd.workloads import (
    WORKLOADS, make_inputs, make_projection_inputs)
from tests._lib import ensure_library, to64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_library()


def _check(got, x, w, b, heads, label):
    from oracle import project
    x64, w64 = to64(x), to64(w)
    b64 = to64(b) if b is not None else None
    refs = project(x64, w64, b64, heads)
    absd = project(np.abs(x64), np.abs(w64), np.abs(b64) if b64 is not None else None, heads)
    D = x.shape[-1]
    g = got.double().cpu().numpy()
    assert g.shape[0] == len(refs)
    for p, (ref, a) in enumerate(zip(refs, absd)):
        e = 4.0 * (D + 1) * 2.0 ** -24 * a
        err = np.abs(g[p] - ref)
        bound = 2.0 ** -8 * (np.abs(ref) + e) + e
        worst = (err / bound).max()
        rel = np.sqrt((err ** 2).mean()) / np.sqrt((ref ** 2).mean())
        print(f"  {label}/p{p}: max err {err.max():.3e}, worst err/bound {worst:.3f}, "
              f"rel-rms {rel:.3e}", flush=True)
        assert np.isfinite(g[p]).all()
        assert worst <= 1.0, f"{label}/p{p}: error above the bound"
        assert rel <= 2.0 ** -8, f"{label}/p{p}: rel-rms {rel:.3e}"


CASES = [
    # B, n, d_model, heads, P, bias
    (1, 300, 128, 2, 3, True),     # ragged token tail, 2 feature tiles per head pair
    (2, 777, 192, 3, 6, False),    # ragged, odd heads: 18 head blocks
    (1, 1, 64, 1, 1, True),        # one token, one head block (half a feature tile)
    (3, 100, 64, 1, 3, True),      # 3 head blocks: the last feature tile half empty
    (2, 256, 1024, 1, 2, True),    # long reduction (16 stages), exact token tiles
    (1, 513, 128, 4, 3, False),    # one token past a tile
    (1, 40, 128, 2, 6, True),      # fewer tokens than one tile
]


@pytest.mark.parametrize("B,n,D,H,P,bias", CASES,
                         ids=[f"B{c[0]}_n{c[1]}_D{c[2]}_H{c[3]}_P{c[4]}" for c in CASES])
def test_project_small(B, n, D, H, P, bias):
    from sliding_window_attention_banded_amd import project
    for seed in (0, 1):
        print(f"[proj] B{B} n{n} D{D} H{H} P{P} bias={bias} seed={seed}", flush=True)
        x, w, b = make_projection_inputs(B, n, D, H, P, seed, bias)
        out = project(x.cuda(), w.cuda(), b.cuda() if b is not None else None, heads=H)
        torch.cuda.synchronize()
        _check(out, x, w, b, H, f"B{B}n{n}D{D}H{H}P{P}s{seed}")


@pytest.mark.parametrize("B,n,D,H,P", [
    (2, 4096, 768, 12, 6),    # Longformer-base encoder layer, local + global projections
    (1, 16384, 768, 12, 6),   # LED encoder layer at 16K tokens
    (4, 4096, 768, 12, 3),    # QA batch, local projections only
    (2, 4096, 768, 12, 3),    # encoder layer without global tokens (256 x 128 workgroup tiles)
])
def test_project_full_size(B, n, D, H, P):
    from sliding_window_attention_banded_amd import project
    print(f"[proj] full B{B} n{n} D{D} H{H} P{P}", flush=True)
    x, w, b = make_projection_inputs(B, n, D, H, P, 0, True)
    out = project(x.cuda(), w.cuda(), b.cuda(), heads=H)
    torch.cuda.synchronize()
    _check(out, x, w, b, H, f"full B{B}n{n}")


def test_project_then_attention_matches_the_oracle_chain():
    """x -> projections -> banded attention with a global token, on the GPU,
    against the oracle's projections (float64) fed to the oracle's attention.
    The GPU attention reads the bf16-rounded projections, so the attention
    tolerance (2e-2 max-abs on O) covers the chain."""
    from oracle import attention, project as oproject
    from sliding_window_attention_banded_amd import Plan, project
    B, n, D, H = 1, 700, 128, 2
    win, dil, G = (64, 32), (1, 2), (0, 350)
    x, w, b = make_projection_inputs(B, n, D, H, 6, 3, True)
    qkv = project(x.cuda(), w.cuda(), b.cuda(), heads=H)
    with Plan(B, H, n, 64, win, dil, False, G, torch.bfloat16) as pl:
        o, lse = pl.forward(*(qkv[i] for i in range(6)), want_lse=True)
    torch.cuda.synchronize()
    t = oproject(to64(x), to64(w), to64(b), H)
    ro, rl = attention(*t, window=list(win), dilation=list(dil), causal=False, global_idx=list(G))
    err = np.abs(o.double().cpu().numpy() - ro).max()
    lerr = np.abs(lse.double().cpu().numpy() - rl).max()
    print(f"  chain: O max-abs {err:.3e}, LSE max-abs {lerr:.3e}", flush=True)
    assert err <= 2e-2 and lerr <= 2e-2


def test_project_rejects_fp16_and_bad_shapes():
    from sliding_window_attention_banded_amd import SwattnError, project
    x = torch.zeros((1, 8, 64), dtype=torch.float16, device="cuda")
    w = torch.zeros((192, 64), dtype=torch.float16, device="cuda")
    with pytest.raises(SwattnError):
        project(x, w, heads=1)
    with pytest.raises(SwattnError):
        project(x.bfloat16(), torch.zeros((100, 64), dtype=torch.bfloat16, device="cuda"), heads=1)


def _draw(i):
    rng = np.random.default_rng(500 + i)
    B = int(rng.integers(1, 4))
    n = int(rng.integers(1, 40)) if rng.random() < 0.2 else int(rng.integers(40, 1500))
    D = 32 * int(rng.integers(1, 33))        # any multiple of 32 up to 1024
    H = int(rng.integers(1, 7))
    P = int(rng.integers(1, 7))
    return B, n, D, H, P, bool(rng.random() < 0.7)


def _draw_large(i):
    # large enough for 256-token workgroups (at least two per CU), ragged
    rng = np.random.default_rng(900 + i)
    B = int(rng.integers(1, 4))
    n = int(rng.integers(8000, 20001)) // B | 1
    D = int(rng.choice([512, 768]))
    H = int(rng.integers(4, 13))
    P = int(rng.integers(3, 7))
    return B, n, D, H, P, bool(rng.random() < 0.7)


RANDOM = [_draw(i) for i in range(32)] + [_draw_large(i) for i in range(4)]


@pytest.mark.parametrize("B,n,D,H,P,bias", RANDOM,
                         ids=[f"r{i}_B{c[0]}_n{c[1]}_D{c[2]}_H{c[3]}_P{c[4]}" for i, c in enumerate(RANDOM)])
def test_project_random_shapes(B, n, D, H, P, bias):
    """Seeded shapes: batch, ragged token counts (1 to 1500, and four large
    ones of 8000 to 20000 tokens), d_model any multiple of 32 up to 1024, 1
    to 12 heads, 1 to 6 projections, with or without bias; the small ones
    run 128-token workgroups, the large ones 256-token workgroups."""
    from sliding_window_attention_banded_amd import project
    print(f"[proj] random B{B} n{n} D{D} H{H} P{P} bias={bias}", flush=True)
    x, w, b = make_projection_inputs(B, n, D, H, P, 11, bias)
    out = project(x.cuda(), w.cuda(), b.cuda() if b is not None else None, heads=H)
    torch.cuda.synchronize()
    _check(out, x, w, b, H, f"rand B{B}n{n}D{D}H{H}P{P}")


# fp32 projections: no final rounding, so the bound is the accumulation's
# alone, |got - ref| <= E = 4 (D+1) 2^-24 A per element, with A as above
# (the vector-ALU kernel sums in input-feature order with fp32 FMAs, whose
# error is at most (D+1) 2^-24 A; 4x as margin).
CASES_F32 = [
    (1, 300, 128, 2, 3, True),
    (2, 777, 192, 3, 6, False),
    (1, 1, 64, 1, 1, True),
    (2, 256, 1024, 1, 2, True),
]


@pytest.mark.parametrize("B,n,D,H,P,bias", CASES_F32,
                         ids=[f"f32_B{c[0]}_n{c[1]}_D{c[2]}_H{c[3]}_P{c[4]}" for c in CASES_F32])
def test_project_fp32(B, n, D, H, P, bias):
    from oracle import project as oracle_project
    from sliding_window_attention_banded_amd import project
    print(f"[proj-f32] B{B} n{n} D{D} H{H} P{P} bias={bias}", flush=True)
    x, w, b = make_projection_inputs(B, n, D, H, P, 3, bias, dtype="fp32")
    out = project(x.cuda(), w.cuda(), b.cuda() if b is not None else None, heads=H)
    torch.cuda.synchronize()
    assert out.dtype == torch.float32
    x64, w64 = to64(x), to64(w)
    b64 = to64(b) if b is not None else None
    refs = oracle_project(x64, w64, b64, H)
    absd = oracle_project(np.abs(x64), np.abs(w64), np.abs(b64) if b64 is not None else None, H)
    g = out.double().cpu().numpy()
    for p, (ref, a) in enumerate(zip(refs, absd)):
        e = 4.0 * (D + 1) * 2.0 ** -24 * a
        err = np.abs(g[p] - ref)
        worst = float((err / (e + 1e-30)).max())
        print(f"  p{p}: max err {err.max():.3e}, worst err/bound {worst:.3f}", flush=True)
        assert np.isfinite(g[p]).all()
        assert worst <= 1.0, f"p{p}: error above the fp32 bound"


def test_project_rejects_mixed_dtypes():
    from sliding_window_attention_banded_amd import SwattnError, project
    x, w, b = make_projection_inputs(1, 64, 64, 1, 1, 0, True, dtype="fp32")
    with pytest.raises(SwattnError):
        project(x.cuda(), w.cuda().to(torch.bfloat16), b.cuda(), heads=1)


def test_project_then_attention_fp32_chain():
    """The fp32 path end to end: x -> fp32 projections -> fp32 banded
    attention with a global token, against the oracle's float64 projections
    fed to its attention, at the fp32 tolerance of the attention (1e-5)."""
    from oracle import attention, project as oproject
    from sliding_window_attention_banded_amd import Plan, project
    B, n, D, H = 1, 512, 128, 2
    win, dil, G = (64, 32), (1, 2), (0, 300)
    x, w, b = make_projection_inputs(B, n, D, H, 6, 4, True, dtype="fp32")
    qkv = project(x.cuda(), w.cuda(), b.cuda(), heads=H)
    with Plan(B, H, n, 64, win, dil, False, G, torch.float32) as pl:
        o, lse = pl.forward(*(qkv[i] for i in range(6)), want_lse=True)
    torch.cuda.synchronize()
    t = oproject(to64(x), to64(w), to64(b), H)
    ro, rl = attention(*t, window=list(win), dilation=list(dil), causal=False, global_idx=list(G))
    err = np.abs(o.double().cpu().numpy() - ro).max()
    lerr = np.abs(lse.double().cpu().numpy() - rl).max()
    print(f"  fp32 chain: O max-abs {err:.3e}, LSE max-abs {lerr:.3e}", flush=True)
    assert err <= 1e-5 and lerr <= 1e-5
