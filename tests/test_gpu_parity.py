"""GPU parity: the HIP library against the float64 oracle, element by element.

Small and ragged shapes are compared in full; the full-size workloads (the
shapes the benchmark times, in the same launch configuration) are compared on
sampled rows that the oracle computes one by one. Each case prints what it
is before it touches the GPU.
"""
import numpy as np
import pytest
import torch

from sliding_window_attention_banded_amd.workloads import (
    WORKLOADS, Workload, global_union, has_globals, make_inputs)
from tests._lib import compare, ensure_library, oracle_ref, run_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_library()


def W(name, B, H, n, window, dilation, causal=False, G=(), dtype="bf16", scale=0.125):
    win = (window,) * H if isinstance(window, int) else tuple(window)
    dil = (dilation,) * H if isinstance(dilation, int) else tuple(dilation)
    return Workload(name, B, H, n, 64, win, dil, causal, tuple(G), dtype, scale)


SMALL = [
    WORKLOADS["single_head_fp32_n512_w64"],
    W("ragged_mix", 2, 3, 1000, (64, 128, 30), (1, 2, 3), False, (0, 17, 999)),
    W("ragged_causal", 1, 4, 777, (32, 256, 2, 1024), (1, 4, 1, 2), True),
    W("ragged_causal_g", 1, 4, 777, (32, 256, 2, 1024), (1, 4, 1, 2), True, (5, 300, 776)),
    W("ragged_mix_fp32", 2, 3, 1000, (64, 128, 30), (1, 2, 3), False, (0, 17, 999), "fp32"),
    W("ragged_causal_fp32", 1, 4, 777, (32, 256, 2, 1024), (1, 4, 1, 2), True, (5, 300), "fp32"),
    W("many_globals", 2, 2, 700, (64, 16), (1, 3), False, tuple(range(0, 700, 7))),
    W("wide_window", 1, 2, 300, (1000, 602), (1, 1), False),
    W("wide_window_causal", 1, 2, 300, (1000, 602), (1, 1), True),
    W("window0", 1, 2, 200, (0, 0), (1, 5), False, (3,)),
    W("dil_beyond_n", 1, 2, 150, (8, 4), (200, 149), False),
    W("all_global", 1, 2, 130, (8, 4), (1, 2), False, tuple(range(130))),
    W("all_global_causal", 1, 1, 130, 8, 1, True, tuple(range(130))),
    # one set of global tokens per batch item (one item with none, one with
    # more than a 64-key tile)
    W("per_item", 3, 2, 700, (64, 16), (1, 3), False, ((0, 5, 699), (), tuple(range(100, 190)))),
    W("per_item_causal", 2, 3, 500, (32, 256, 2), (1, 4, 1), True, ((7,), (0, 250, 499))),
    # one global token per item (the headline's and LED's case)
    W("one_global", 2, 3, 1000, (64, 128, 30), (1, 2, 3), False, (17,)),
    W("one_global_causal", 1, 4, 777, (32, 256, 2, 1024), (1, 4, 1, 2), True, (300,)),
    W("one_global_fp32", 2, 3, 1000, (64, 128, 30), (1, 2, 3), False, (999,), "fp32"),
    W("one_global_per_item", 3, 2, 700, (64, 16), (1, 3), False, ((5,), (), (699,))),
    W("one_global_per_item_causal", 2, 2, 2100, (32, 256), (1, 4), True, ((0,), (2050,))),
]

EDGE_N = [1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255]


def _case(wl, seed, kind, rows=None):
    print(f"[parity] {wl.name} B{wl.batch} H{wl.heads} n{wl.n} {wl.dtype} "
          f"causal={wl.causal} |G|={len(wl.global_idx)} seed={seed} kind={kind}", flush=True)
    inp = make_inputs(wl, seed, kind)
    o, lse = run_gpu(wl, inp)
    ref_o, ref_lse = oracle_ref(wl, inp, rows=rows)
    return compare(wl, o, lse, ref_o, ref_lse, rows=rows, label=wl.name)


@pytest.mark.parametrize("wl", SMALL, ids=lambda w: w.name)
@pytest.mark.parametrize("kind", ["normal", "sharp"])
def test_small_full_compare(wl, kind):
    for seed in (0, 1, 2):
        _case(wl, seed, kind)


@pytest.mark.parametrize("wl", [w for w in SMALL if has_globals(w)], ids=lambda w: w.name)
def test_small_dedup(wl):
    _case(wl, 0, "dedup")


@pytest.mark.parametrize("n", EDGE_N)
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("causal", [False, True])
def test_edge_lengths(n, dtype, causal):
    G = (0, n - 1) if n > 2 else ()
    wl = W(f"edge_n{n}", 1, 3, n, (6, 64, 0), (1, 2, 7), causal, G, dtype)
    _case(wl, n, "sharp")


def _sample_rows(wl, count=48, seed=0):
    n = wl.n
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 2, 31, 32, 63, 64, 127, 128, 129, 255, 256, 257, 300, 319, 320,
             511, 512, 513, n // 2, n - 300, n - 257, n - 256, n - 129, n - 128,
             n - 65, n - 64, n - 33, n - 32, n - 2, n - 1]
    rows = set(r for r in fixed if 0 <= r < n)
    gu = global_union(wl)
    rows |= set(int(x) for x in gu[:4]) | set(int(x) for x in gu[-2:])
    rows |= set(int(x) for x in rng.integers(0, n, count))
    return np.array(sorted(rows))


FULL = ["encoder_b2_h12_n4096_w512_g1", "encoder_b2_h12_n4096_w512",
        "arlm_b1_h12_n8192_w512_causal_dil2", "arlm_b1_h8_n23040_w1024_causal_dil4",
        "qa_b4_h12_n4096_w512_g64", "qa_b4_h12_n4096_w512_gper", "led_b1_h12_n16384_w1024_g1",
        "led_decoder_b1_h12_n1024_causal"]


@pytest.mark.parametrize("name", FULL)
@pytest.mark.parametrize("kind", ["normal", "sharp", "dedup"])
def test_full_size_sampled_rows(name, kind):
    wl = WORKLOADS[name]
    if kind == "dedup" and not has_globals(wl):
        pytest.skip("dedup inputs need global tokens")
    _case(wl, 0, kind, rows=_sample_rows(wl))


@pytest.mark.parametrize("name", ["encoder_b2_h12_n4096_w512_g1", "encoder_b2_h12_n4096_w512",
                                  "arlm_b1_h12_n8192_w512_causal_dil2", "qa_b4_h12_n4096_w512_g64"])
@pytest.mark.parametrize("kind", ["sharp", "dedup"])
def test_full_size_whole_tensors(name, kind):
    """Every row of every (batch, head) of the full-size workloads, in the
    launch configuration the benchmark times."""
    wl = WORKLOADS[name]
    if kind == "dedup" and not has_globals(wl):
        pytest.skip("dedup inputs need global tokens")
    _case(wl, 0, kind)


@pytest.mark.parametrize("name,bh", [
    ("arlm_b1_h8_n23040_w1024_causal_dil4", (0, 0)),   # dilation 1
    ("arlm_b1_h8_n23040_w1024_causal_dil4", (0, 7)),   # dilation 4
    ("led_b1_h12_n16384_w1024_g1", (0, 0)),
    ("led_b1_h12_n16384_w1024_g1", (0, 11)),
])
@pytest.mark.parametrize("kind", ["sharp", "normal"])
def test_full_size_whole_slices(name, bh, kind):
    """Whole (batch, head) slices of the two longest workloads: every row of
    the slice against the oracle on that slice alone."""
    wl = WORKLOADS[name]
    b, h = bh
    print(f"[parity] {wl.name} slice {bh} kind={kind}", flush=True)
    inp = make_inputs(wl, 0, kind)
    o, lse = run_gpu(wl, inp)
    one = wl.with_(name=f"{wl.name}[{b},{h}]", batch=1, heads=1, window=(wl.window[h],),
                   dilation=(wl.dilation[h],),
                   global_idx=tuple(global_union(wl)) if has_globals(wl) else ())
    sl = {k: (v[b:b + 1, h:h + 1] if v is not None else None) for k, v in inp.items()}
    ref_o, ref_lse = oracle_ref(one, sl)
    compare(one, o[b:b + 1, h:h + 1], lse[b:b + 1, h:h + 1], ref_o, ref_lse, label=one.name)


# Several global tokens in long sequences: the global rows' keys come in
# more than 16 chunks (9000 keys in 256-key chunks: 36), so the merge folds
# them in batches of 16 with a ragged last batch.
LONG_G = [
    W("long_globals", 1, 2, 9000, (64, 128), (1, 2), False, (0, 4500, 8999)),
    W("long_globals_causal", 1, 2, 9000, (64, 128), (1, 2), True, (3, 4500, 8999)),
    W("long_globals_fp32", 1, 1, 9000, 64, 1, False, (0, 8999), "fp32"),
    W("long_globals_per_item", 2, 1, 9000, 64, 1, False, ((0, 8999), (4500,))),
]


@pytest.mark.parametrize("wl", LONG_G, ids=lambda w: w.name)
@pytest.mark.parametrize("kind", ["normal", "sharp"])
def test_long_sequence_global_rows(wl, kind):
    _case(wl, 0, kind, rows=_sample_rows(wl))


def test_full_size_headline_all_seeds():
    wl = WORKLOADS["encoder_b2_h12_n4096_w512_g1"]
    for seed in (1, 2):
        _case(wl, seed, "sharp", rows=_sample_rows(wl, seed=seed))


@pytest.mark.parametrize("wl", SMALL, ids=lambda w: w.name)
@pytest.mark.parametrize("key_split", [1, 3, 8])
def test_key_split_forced(wl, key_split):
    """The band keys of every tile shared out over 1 (no split), 3 or 8
    workgroups, merged afterwards: the same result within the tolerances
    (small problems otherwise choose their split themselves)."""
    from sliding_window_attention_banded_amd import Plan
    print(f"[parity] {wl.name} key_split={key_split}", flush=True)
    inp = make_inputs(wl, 0, "sharp")
    with Plan(wl.batch, wl.heads, wl.n, wl.d, wl.window, wl.dilation, wl.causal,
              wl.global_idx, wl.torch_dtype, key_split=key_split) as pl:
        o, lse = run_gpu(wl, inp, plan=pl)
    ref_o, ref_lse = oracle_ref(wl, inp)
    compare(wl, o, lse, ref_o, ref_lse, label=f"{wl.name}/split{key_split}")


@pytest.mark.parametrize("G", [(0,), ((3,), (), (1500,))], ids=["shared", "per_item"])
def test_repeated_launches_one_global(G):
    """Back-to-back forwards on one plan, each checked: every launch reuses
    the plan's global-row workspace (the chunk partials and their merge), so
    nothing a launch leaves there may leak into the next one."""
    wl = W("repeat_one_global", 3 if len(G) == 3 else 2, 3, 1600, (64, 128, 30), (1, 2, 3),
           False, G)
    from sliding_window_attention_banded_amd import Plan
    print(f"[parity] {wl.name} G={G}: 6 launches on one plan", flush=True)
    with Plan(wl.batch, wl.heads, wl.n, wl.d, wl.window, wl.dilation, wl.causal,
              wl.global_idx, wl.torch_dtype, key_split=1) as pl:
        ins, outs = [], []
        for seed in range(6):
            inp = make_inputs(wl, 100 + seed, "sharp" if seed % 2 else "normal")
            dev = {k: (v.cuda() if v is not None else None) for k, v in inp.items()}
            outs.append(pl.forward(dev["q"], dev["k"], dev["v"], dev["qg"], dev["kg"],
                                   dev["vg"], want_lse=True))
            ins.append(inp)
        torch.cuda.synchronize()
        for seed, (inp, (o, lse)) in enumerate(zip(ins, outs)):
            ref_o, ref_lse = oracle_ref(wl, inp)
            compare(wl, o.cpu(), lse.cpu(), ref_o, ref_lse, label=f"launch {seed}")


ONE_GLOBAL = [w for w in SMALL if w.name.startswith("one_global")]


@pytest.mark.parametrize("wl", ONE_GLOBAL, ids=lambda w: w.name)
@pytest.mark.parametrize("kind", ["normal", "sharp"])
def test_one_global_no_key_split(wl, kind):
    """One global token and no key split (the headline's launch
    configuration), whatever split the plan would choose for these shapes."""
    from sliding_window_attention_banded_amd import Plan
    with Plan(wl.batch, wl.heads, wl.n, wl.d, wl.window, wl.dilation, wl.causal,
              wl.global_idx, wl.torch_dtype, key_split=1) as pl:
        for seed in (0, 1):
            print(f"[parity] {wl.name} key_split=1 seed={seed} kind={kind}", flush=True)
            inp = make_inputs(wl, seed, kind)
            o, lse = run_gpu(wl, inp, plan=pl)
            ref_o, ref_lse = oracle_ref(wl, inp)
            compare(wl, o, lse, ref_o, ref_lse, label=wl.name)


def test_tensors_past_two_gib():
    """Every [B, H, n, 64] tensor larger than 2 GiB (18 heads of 2^20 + 3
    tokens): rows of the first and of the last head (whose data lies past
    2^31 bytes), band rows near both ends, the global rows and random rows,
    against the oracle on that head alone."""
    from sliding_window_attention_banded_amd import Plan
    from sliding_window_attention_banded_amd.workloads import make_device_inputs
    n, H = (1 << 20) + 3, 18
    wl = W("past_2gib", 1, H, n, 64, [1] * 16 + [3, 1], False, (7, n - 1))
    assert H * n * 64 * 2 > (1 << 31)
    print(f"[parity] {wl.name} B1 H{H} n{n} (sharp, drawn on the device)", flush=True)
    dev = make_device_inputs(wl, 5, "cuda")
    with Plan(wl.batch, wl.heads, wl.n, wl.d, wl.window, wl.dilation, wl.causal,
              wl.global_idx, wl.torch_dtype) as pl:
        o, lse = pl.forward(dev["q"], dev["k"], dev["v"], dev["qg"], dev["kg"], dev["vg"],
                            want_lse=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(11)
    rows = np.array(sorted({0, 1, 7, 40, n // 2, n - 40, n - 2, n - 1}
                           | set(rng.integers(0, n, 6).tolist())))
    for h in (0, H - 2, H - 1):
        one = W("past_2gib_head", 1, 1, n, wl.window[h], wl.dilation[h], False, (7, n - 1))
        inp = {k: (v[:, h:h + 1].cpu() if v is not None else None) for k, v in dev.items()}
        ref_o, ref_lse = oracle_ref(one, inp, rows=rows)
        compare(one, o[:, h:h + 1].cpu(), lse[:, h:h + 1].cpu(), ref_o, ref_lse, rows=rows,
                label=f"{wl.name}/head{h}")
