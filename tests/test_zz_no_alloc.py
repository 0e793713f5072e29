"""The allocation-free forward (swattn_forward_noalloc) against the plan-based
forward (swattn_create + swattn_forward), through the C ABI.

Both run the same kernels on the same inputs; only where their tables and
partial results live differs (a static device array instead of the plan's
allocation), so O and LSE must agree bit for bit. Two calls in a row share
that array: the second, on a smaller problem, must not see the first one's
contents. Each case prints what it is before it touches the GPU.
"""
import ctypes

import pytest
import torch

from sliding_window_attention_banded_amd import Plan, binding, forward_noalloc
from sliding_window_attention_banded_amd.workloads import Workload, make_inputs
from tests._lib import compare, ensure_library, oracle_ref

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_library()


# The first problem uses every piece of the array: per-head geometry (a tile
# list), global tokens (global-row partials). The second is smaller and small
# enough that the library shares each tile's keys over two workgroups (key-
# split partials), with per-item global sets and the causal mask.
FIRST = Workload("noalloc_first", 2, 3, 1500, 64, (64, 256, 30), (1, 2, 3), False,
                 (0, 17, 700, 1499))
SECOND = Workload("noalloc_second", 2, 2, 300, 64, (256, 256), (1, 1), True,
                  ((0, 5), (299,)))


def _dev(inp):
    return {k: (v.cuda() if v is not None else None) for k, v in inp.items()}


def _plan_forward(wl, d):
    with Plan(wl.batch, wl.heads, wl.n, wl.d, wl.window, wl.dilation, wl.causal,
              wl.global_idx, wl.torch_dtype) as pl:
        o, lse = pl.forward(d["q"], d["k"], d["v"], d["qg"], d["kg"], d["vg"], want_lse=True)
        torch.cuda.synchronize()
    return o, lse


def _noalloc_forward(wl, d):
    o, lse = forward_noalloc(d["q"], d["k"], d["v"], d["qg"], d["kg"], d["vg"],
                             window=list(wl.window), dilation=list(wl.dilation),
                             causal=wl.causal, global_idx=wl.global_idx, want_lse=True)
    torch.cuda.synchronize()
    return o, lse


def test_two_calls_match_the_plan_forward():
    results = []
    for wl, seed in ((FIRST, 0), (SECOND, 1)):
        print(f"[noalloc] {wl.name}: B{wl.batch} H{wl.heads} n{wl.n}", flush=True)
        inp = make_inputs(wl, seed, "sharp")
        d = _dev(inp)
        o_ref, l_ref = _plan_forward(wl, d)
        o, lse = _noalloc_forward(wl, d)
        assert torch.equal(o, o_ref), f"{wl.name}: O differs from the plan-based forward"
        assert torch.equal(lse, l_ref), f"{wl.name}: LSE differs from the plan-based forward"
        results.append((wl, inp, o.cpu(), lse.cpu()))
    # and both against the float64 oracle
    for wl, inp, o, lse in results:
        ref_o, ref_l = oracle_ref(wl, inp)
        compare(wl, o, lse, ref_o, ref_l, label=wl.name)


# One global token per item and no key split: the global row is streamed in
# chunks whose last block folds them, counting arrivals per (batch, head) in
# the array; the counters must start every call at zero. Two calls in a row,
# the second smaller, each bit-identical to the plan's forward.
ONE_G = (Workload("noalloc_one_global", 2, 2, 2000, 64, (128, 128), (1, 1), False, (17,)),
         Workload("noalloc_one_global_small", 1, 2, 900, 64, (64, 64), (1, 1), True, ((600,),)))


def test_one_global_token_folded_in_the_kernel():
    for wl, seed in ((ONE_G[0], 2), (ONE_G[1], 3)):
        print(f"[noalloc] {wl.name}: B{wl.batch} H{wl.heads} n{wl.n}", flush=True)
        inp = make_inputs(wl, seed, "normal")
        d = _dev(inp)
        o_ref, l_ref = _plan_forward(wl, d)
        o, lse = _noalloc_forward(wl, d)
        assert torch.equal(o, o_ref), f"{wl.name}: O differs from the plan-based forward"
        assert torch.equal(lse, l_ref), f"{wl.name}: LSE differs from the plan-based forward"
        ref_o, ref_l = oracle_ref(wl, inp)
        compare(wl, o.cpu(), lse.cpu(), ref_o, ref_l, label=wl.name)


def test_a_problem_beyond_the_array_is_rejected():
    # global-row partials alone: 64 heads x 4096 tokens x 4096 chunks of
    # 256 keys... far above the 32 MiB array; rejected before any launch
    print("[noalloc] oversized problem", flush=True)
    lib = binding.load_library()
    heads, n = 64, 1 << 20
    ps = binding._ParamSet(1, heads, n, 64, 512, 1, False, tuple(range(64)), torch.bfloat16, 0)
    fake = ctypes.c_void_p(1 << 20)  # aligned, never dereferenced: the call fails first
    status = lib.swattn_forward_noalloc(ctypes.byref(ps.params), fake, fake, fake, fake, fake,
                                        fake, ctypes.c_void_p(1 << 40), None, None)
    assert status == binding.ERR_UNSUPPORTED
    assert b"scratch" in lib.swattn_last_error()
