"""Workload shapes and seeded synthetic inputs.

This module holds no arithmetic of the attention method: it only names shapes
and draws random tensors. Both the HIP path (tests, bench) and the float64
oracle consume what it produces, so it is the one module they share.

Shapes stand in for the workloads on the Longformer summary page: the
Longformer-base encoder shape, the autoregressive character-LM shapes of
section 4 (windows per layer, dilation on two heads, staged sequence length up
to 23,040), the QA shape of section 3-1 "Global Attention" (question tokens as
globals) and the LED encoder of section 7 (16K tokens, window 1024, one global
token) with its decoder's left-only self-attention. No dataset is read; every
tensor is drawn from a seeded generator.
"""

from __future__ import annotations

from dataclasses import dataclass, field, replace

import torch

__all__ = ["Workload", "WORKLOADS", "make_inputs", "DTYPES", "item_globals", "has_globals",
           "global_union", "make_projection_inputs"]

DTYPES = {"bf16": torch.bfloat16, "fp32": torch.float32}


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int
    n: int
    d: int
    window: tuple
    dilation: tuple
    causal: bool
    # one set of global positions for every batch item, or (per-example
    # global tokens) a tuple of B such sets
    global_idx: tuple = field(default=())
    dtype: str = "bf16"
    scale: float = 0.125

    @property
    def torch_dtype(self):
        return DTYPES[self.dtype]

    def with_(self, **kw):
        return replace(self, **kw)


def item_globals(wl):
    """The global positions of each batch item (a list of B tuples)."""
    g = tuple(wl.global_idx)
    if g and all(isinstance(x, (tuple, list)) for x in g):
        if len(g) != wl.batch:
            raise ValueError("per-example global_idx needs one set per batch item")
        return [tuple(x) for x in g]
    return [g] * wl.batch


def has_globals(wl):
    return any(len(x) for x in item_globals(wl))


def global_union(wl):
    return sorted(set(x for g in item_globals(wl) for x in g))


def _per_head(h, v, over=None):
    t = [v] * h
    for idx, val in (over or {}).items():
        t[idx] = val
    return tuple(t)


WORKLOADS = {
    # single head, fp32, symmetric +-32 window; the small case the oracle
    # finishes in well under a second
    "single_head_fp32_n512_w64": Workload(
        "single_head_fp32_n512_w64", 1, 1, 512, 64, (64,), (1,), False, (),
        "fp32", 8 ** -0.5),
    # Longformer-base-shaped encoder with one global token (position 0)
    "encoder_b2_h12_n4096_w512_g1": Workload(
        "encoder_b2_h12_n4096_w512_g1", 2, 12, 4096, 64, _per_head(12, 512),
        _per_head(12, 1), False, (0,)),
    # the same encoder with no global token: the band pass alone
    "encoder_b2_h12_n4096_w512": Workload(
        "encoder_b2_h12_n4096_w512", 2, 12, 4096, 64, _per_head(12, 512),
        _per_head(12, 1), False, ()),
    # autoregressive char-LM phase: causal, dilation 2 on heads 10-11
    "arlm_b1_h12_n8192_w512_causal_dil2": Workload(
        "arlm_b1_h12_n8192_w512_causal_dil2", 1, 12, 8192, 64,
        _per_head(12, 512), _per_head(12, 1, {10: 2, 11: 2}), True, ()),
    # autoregressive char-LM final stage: n = 23040, dilation 4 on heads 6-7
    "arlm_b1_h8_n23040_w1024_causal_dil4": Workload(
        "arlm_b1_h8_n23040_w1024_causal_dil4", 1, 8, 23040, 64,
        _per_head(8, 1024), _per_head(8, 1, {6: 4, 7: 4}), True, ()),
    # QA-style: 64 global tokens (positions 0-63)
    "qa_b4_h12_n4096_w512_g64": Workload(
        "qa_b4_h12_n4096_w512_g64", 4, 12, 4096, 64, _per_head(12, 512),
        _per_head(12, 1), False, tuple(range(64))),
    # QA-style with per-example questions: item b's first L_b tokens are its
    # global tokens, L = (64, 48, 24, 96)
    "qa_b4_h12_n4096_w512_gper": Workload(
        "qa_b4_h12_n4096_w512_gper", 4, 12, 4096, 64, _per_head(12, 512),
        _per_head(12, 1), False, tuple(tuple(range(L)) for L in (64, 48, 24, 96))),
    # LED encoder: 16K tokens, window 1024, global attention on the first token
    "led_b1_h12_n16384_w1024_g1": Workload(
        "led_b1_h12_n16384_w1024_g1", 1, 12, 16384, 64, _per_head(12, 1024),
        _per_head(12, 1), False, (0,)),
    # LED decoder self-attention: left-only over 1024 output tokens, every
    # earlier token visible (a causal window of 2n covers the whole prefix)
    "led_decoder_b1_h12_n1024_causal": Workload(
        "led_decoder_b1_h12_n1024_causal", 1, 12, 1024, 64, _per_head(12, 2048),
        _per_head(12, 1), True, ()),
}


def _draw(gen, shape, scale, kind, role):
    if kind == "sharp" and role == "v":
        x = torch.rand(shape, generator=gen, dtype=torch.float32) * 2.0 - 1.0
    elif kind == "sharp":
        x = torch.randn(shape, generator=gen, dtype=torch.float32) * 2.0
    else:
        x = torch.randn(shape, generator=gen, dtype=torch.float32) * scale
    return x


def make_inputs(wl: Workload, seed: int, kind: str = "normal"):
    """Seeded CPU tensors q, k, v, qg, kg, vg ([B,H,n,d], the workload dtype).

    Draw order: q, k, v, then qg, kg, vg when the workload has global tokens
    (those three are None otherwise). Values are drawn in float32 and rounded
    to nearest-even into the workload dtype.

    ``kind``:
      * "normal": i.i.d. N(0,1) * scale;
      * "sharp":  q, k ~ N(0,1) * 2 and v ~ U(-1, 1), so softmax rows are
        peaked and a wrong key set moves the output far beyond tolerance;
      * "dedup":  "normal", plus a direction u shared by every query and by the
        regular keys at up to four global positions (every len(G)//4-th of
        the union of the items' sets), with
        one-hot values at those positions: each such key then takes a large
        share of every row, so counting it twice (when it also lies inside a
        row's window) moves the output far beyond tolerance.
    """
    if kind not in ("normal", "sharp", "dedup"):
        raise ValueError(kind)
    gen = torch.Generator(device="cpu").manual_seed(int(seed))
    shape = (wl.batch, wl.heads, wl.n, wl.d)
    out = {}
    roles = ["q", "k", "v"] + (["qg", "kg", "vg"] if has_globals(wl) else [])
    for r in roles:
        out[r] = _draw(gen, shape, wl.scale, kind,
                       "v" if r in ("v", "vg") else "qk")
    if kind == "dedup" and has_globals(wl):
        u = torch.randn((wl.d,), generator=gen, dtype=torch.float32)
        u = u / u.norm() * wl.d ** 0.5
        gu = global_union(wl)
        step = max(1, len(gu) // 4)
        gi = torch.tensor(gu[::step], dtype=torch.long)
        out["q"] = out["q"] + 0.25 * u
        out["k"][:, :, gi, :] = 3.0 * u
        vv = torch.zeros((len(gi), wl.d), dtype=torch.float32)
        vv[torch.arange(len(gi)), torch.arange(len(gi)) % wl.d] = 1.0
        out["v"][:, :, gi, :] = vv
    for r in list(out):
        out[r] = out[r].to(wl.torch_dtype).contiguous()
    for r in ("qg", "kg", "vg"):
        out.setdefault(r, None)
    return out


def make_device_inputs(wl: Workload, seed: int, device, kind: str = "sharp"):
    """The "sharp" (q, k ~ N(0,1) * 2, v ~ U(-1, 1)) or "normal" (every
    tensor N(0,1) * scale) distribution of make_inputs, for q, k, v and, when
    the workload has global tokens, qg, kg, vg, drawn directly on ``device``
    with its own seeded generator: for shapes too large to draw on the host
    (several GB per tensor) and for benchmark input sets. Rounded to
    nearest-even into the workload dtype. (The draws differ from
    make_inputs', which come from a CPU generator.)"""
    if kind not in ("normal", "sharp"):
        raise ValueError(kind)
    gen = torch.Generator(device=device).manual_seed(int(seed))
    shape = (wl.batch, wl.heads, wl.n, wl.d)
    out = {}
    roles = ["q", "k", "v"] + (["qg", "kg", "vg"] if has_globals(wl) else [])
    for r in roles:
        if kind == "normal":
            t = torch.randn(shape, generator=gen, device=device, dtype=torch.float32) * wl.scale
        elif r in ("v", "vg"):
            t = torch.rand(shape, generator=gen, device=device, dtype=torch.float32) * 2.0 - 1.0
        else:
            t = torch.randn(shape, generator=gen, device=device, dtype=torch.float32) * 2.0
        out[r] = t.to(wl.torch_dtype)
        del t
    for r in ("qg", "kg", "vg"):
        out.setdefault(r, None)
    return out


def make_projection_inputs(batch, n, d_model, heads, nproj, seed, bias=True, dtype="bf16"):
    """Seeded CPU tensors for the projections in front of the attention:
    x [batch, n, d_model] ~ N(0, 1) (a normalised layer input), weight
    [nproj*heads*64, d_model] ~ N(0, 1/d_model) (the usual fan-in scaling,
    so that the projections come out of order one) and bias
    [nproj*heads*64] ~ N(0, 0.1^2) or None. Draw order: x, weight, bias;
    drawn in float32 and, for dtype "bf16", rounded to nearest-even bf16."""
    if dtype not in ("bf16", "fp32"):
        raise ValueError(dtype)
    gen = torch.Generator(device="cpu").manual_seed(20_000 + int(seed))
    N = nproj * heads * 64
    x = torch.randn((batch, n, d_model), generator=gen, dtype=torch.float32)
    w = torch.randn((N, d_model), generator=gen, dtype=torch.float32) / d_model ** 0.5
    b = torch.randn((N,), generator=gen, dtype=torch.float32) * 0.1 if bias else None
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    cv = lambda t: None if t is None else t.to(tdt).contiguous()
    return cv(x), cv(w), cv(b)
