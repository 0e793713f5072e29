"""GPU invariants and ABI behaviour that hold at any size, checked through the
C ABI: constant values, projection separation, guard bytes around the output,
determinism, optional LSE, and the error codes of forward."""
import ctypes

import pytest
import torch

from sliding_window_attention_banded_amd import Plan, SwattnError, binding
from sliding_window_attention_banded_amd.workloads import WORKLOADS, Workload, make_inputs
from tests._lib import ensure_library, run_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_library()


WL = Workload("inv", 2, 3, 1500, 64, (64, 128, 512), (1, 3, 1), False, (0, 5, 700, 1499))
WLC = Workload("inv_causal", 1, 4, 2100, 64, (512, 64, 256, 2), (1, 2, 4, 1), True, (3, 1000))


@pytest.mark.parametrize("wl", [WL, WLC, WL.with_(dtype="fp32", name="inv_fp32")],
                         ids=lambda w: w.name)
def test_constant_values_give_constant_output(wl):
    print(f"[inv] constant V {wl.name}", flush=True)
    inp = make_inputs(wl, 0, "sharp")
    c = torch.linspace(-0.9, 0.9, 64).to(wl.torch_dtype)
    inp["v"] = c.expand_as(inp["v"]).contiguous()
    if inp["vg"] is not None:
        inp["vg"] = c.expand_as(inp["vg"]).contiguous()
    o, _ = run_gpu(wl, inp)
    # softmax weights sum to one: only the rounding of P (bf16), of the fp32
    # sums over up to ~10^3 keys and of O moves it (the parity tolerances)
    tol = 1e-2 if wl.dtype == "bf16" else 1e-5
    err = float((o.float() - c.float()).abs().max())
    assert err <= tol, f"{wl.name}: constant-V error {err:.3e}"


@pytest.mark.parametrize("wl", [WL, WLC], ids=lambda w: w.name)
def test_projection_separation_is_exact(wl):
    print(f"[inv] separation {wl.name}", flush=True)
    inp = make_inputs(wl, 1)
    o1, l1 = run_gpu(wl, inp)
    G = list(wl.global_idx)
    reg = [i for i in range(wl.n) if i not in set(G)]
    inp2 = dict(inp)
    inp2["qg"] = -inp["qg"]
    inp2["kg"] = inp["kg"] * 2
    inp2["vg"] = inp["vg"] + 1
    o2, l2 = run_gpu(wl, inp2)
    assert torch.equal(o1[:, :, reg], o2[:, :, reg])
    assert torch.equal(l1[:, :, reg], l2[:, :, reg])
    assert not torch.equal(o1[:, :, G], o2[:, :, G])
    inp3 = dict(inp)
    for t in ("q", "k", "v"):
        x = inp[t].clone()
        x[:, :, reg] = -x[:, :, reg]
        inp3[t] = x
    o3, _ = run_gpu(wl, inp3)
    assert torch.equal(o1[:, :, G], o3[:, :, G])


def test_guard_bytes_determinism_and_optional_lse():
    wl = WL
    print("[inv] guards", flush=True)
    inp = {k: (v.cuda() if v is not None else None) for k, v in make_inputs(wl, 2).items()}
    numel = wl.batch * wl.heads * wl.n * 64
    pad = 4096
    buf = torch.full((numel + 2 * pad,), 7.0, dtype=torch.bfloat16, device="cuda")
    out = buf[pad:pad + numel].view(wl.batch, wl.heads, wl.n, 64)
    lbuf = torch.full((wl.batch * wl.heads * wl.n + 2 * pad,), 7.0, device="cuda")
    lse = lbuf[pad:pad + wl.batch * wl.heads * wl.n].view(wl.batch, wl.heads, wl.n)
    with Plan(wl.batch, wl.heads, wl.n, 64, wl.window, wl.dilation, wl.causal,
              wl.global_idx, torch.bfloat16) as pl:
        pl.forward(inp["q"], inp["k"], inp["v"], inp["qg"], inp["kg"], inp["vg"], out=out, lse=lse)
        o_again, _ = pl.forward(inp["q"], inp["k"], inp["v"], inp["qg"], inp["kg"], inp["vg"])
        o_nolse, none = pl.forward(inp["q"], inp["k"], inp["v"], inp["qg"], inp["kg"], inp["vg"])
        torch.cuda.synchronize()
    assert none is None
    assert (buf[:pad] == 7).all() and (buf[pad + numel:] == 7).all()
    assert (lbuf[:pad] == 7).all() and (lbuf[-pad:] == 7).all()
    assert torch.equal(out, o_again) and torch.equal(out, o_nolse)


def test_forward_error_codes():
    wl = WORKLOADS["encoder_b2_h12_n4096_w512_g1"].with_(batch=1, heads=1, n=256)
    print("[inv] error codes", flush=True)
    inp = {k: v.cuda() for k, v in make_inputs(wl, 0).items()}
    lib = binding.load_library()
    with Plan(1, 1, 256, 64, 512, 1, False, (0,), torch.bfloat16) as pl:
        q, k, v, qg, kg, vg = (inp[x].data_ptr() for x in ("q", "k", "v", "qg", "kg", "vg"))
        o = torch.empty_like(inp["q"])
        h = pl._h
        fwd = lib.swattn_forward
        assert fwd(h, q, k, v, qg, kg, vg, o.data_ptr(), None, None) == 0
        assert fwd(h, q, k, v, None, kg, vg, o.data_ptr(), None, None) == binding.ERR_INVALID_ARG
        assert fwd(h, q, k, v, qg, kg, vg, q, None, None) == binding.ERR_INVALID_ARG
        assert fwd(h, q, k, v, qg, kg, vg, o.data_ptr() + 8, None, None) == binding.ERR_ALIGNMENT
        assert fwd(h, q + 2, k, v, qg, kg, vg, o.data_ptr(), None, None) == binding.ERR_ALIGNMENT
        assert fwd(h, None, k, v, qg, kg, vg, o.data_ptr(), None, None) == binding.ERR_INVALID_ARG
        torch.cuda.synchronize()
    with Plan(1, 1, 256, 64, 512, 1, False, (), torch.bfloat16) as pl2:
        with pytest.raises(SwattnError):
            pl2.forward(inp["q"], inp["k"], inp["v"], inp["qg"], inp["kg"], inp["vg"])
        with pytest.raises(SwattnError):
            pl2.forward(inp["q"].float(), inp["k"], inp["v"])
    torch.cuda.synchronize()


def test_plans_on_two_streams_give_identical_results():
    wl = WLC
    print("[inv] streams", flush=True)
    inp = {k: (v.cuda() if v is not None else None) for k, v in make_inputs(wl, 3).items()}
    args = (wl.batch, wl.heads, wl.n, 64, wl.window, wl.dilation, wl.causal, wl.global_idx)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    with Plan(*args) as p1, Plan(*args) as p2:
        torch.cuda.synchronize()
        with torch.cuda.stream(s1):
            a, _ = p1.forward(inp["q"], inp["k"], inp["v"], inp["qg"], inp["kg"], inp["vg"])
        with torch.cuda.stream(s2):
            b, _ = p2.forward(inp["q"], inp["k"], inp["v"], inp["qg"], inp["kg"], inp["vg"])
        torch.cuda.synchronize()
    assert torch.equal(a, b)
