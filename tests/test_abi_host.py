"""The C-ABI library loads, exports every declared entry point, and rejects
bad parameters on the host before touching a device (no compute here)."""
import ctypes

import pytest

from sliding_window_attention_banded_amd import binding
from tests._lib import declared_functions, ensure_library


@pytest.fixture(scope="module")
def lib():
    return ensure_library()


def test_header_declares_the_abi():
    assert declared_functions() == sorted(binding.EXPORTS)


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    names = [lib.swattn_status_string(i).decode() for i in range(5)]
    assert names == ["SWATTN_OK", "SWATTN_ERR_INVALID_ARG", "SWATTN_ERR_UNSUPPORTED",
                     "SWATTN_ERR_HIP", "SWATTN_ERR_ALIGNMENT"]
    assert lib.swattn_status_string(99).decode() == "SWATTN_UNKNOWN_STATUS"


def _params(**kw):
    heads = kw.get("heads", 2)
    win = (ctypes.c_int32 * heads)(*kw.get("window", [4] * heads))
    dil = (ctypes.c_int32 * heads)(*kw.get("dilation", [1] * heads))
    gl = kw.get("global_idx", [])
    G = (ctypes.c_int32 * max(1, len(gl)))(*gl)
    offs = kw.get("offsets")
    O = (ctypes.c_int32 * len(offs))(*offs) if offs is not None else None
    p = binding._Params(kw.get("batch", 1), heads, kw.get("n", 16), kw.get("d", 64),
                        win, dil, kw.get("causal", 0),
                        ctypes.cast(G, ctypes.POINTER(ctypes.c_int32)),
                        kw.get("n_global", len(gl)), kw.get("dtype", 0),
                        ctypes.cast(O, ctypes.POINTER(ctypes.c_int32)) if O is not None else None,
                        kw.get("key_split", 0))
    return p, (win, dil, G, O)


@pytest.mark.parametrize("kw,code", [
    (dict(batch=0), 1), (dict(heads=0, window=[], dilation=[]), 1),
    (dict(n=0), 1), (dict(n=(1 << 24) + 1), 1), (dict(causal=2), 1),
    (dict(window=[3, 4]), 1), (dict(window=[-2, 4]), 1), (dict(dilation=[0, 1]), 1),
    (dict(global_idx=[3, 3]), 1), (dict(global_idx=[16]), 1),
    (dict(global_idx=[-1]), 1), (dict(n_global=17), 1), (dict(d=128), 2),
    (dict(dtype=7), 2), (dict(key_split=-1), 1), (dict(key_split=17), 1),
    # per-example sets: offsets must start at 0, end at n_global, not decrease;
    # each item's set in [0, n), no repeats within an item, at most n entries
    (dict(batch=2, global_idx=[1, 2], offsets=[1, 1, 2]), 1),
    (dict(batch=2, global_idx=[1, 2], offsets=[0, 1, 3], n_global=2), 1),
    (dict(batch=2, global_idx=[1, 2], offsets=[0, 2, 1], n_global=2), 1),
    (dict(batch=2, global_idx=[1, 1], offsets=[0, 2, 2]), 1),
    (dict(batch=2, global_idx=[1, 16], offsets=[0, 1, 2]), 1),
    (dict(batch=2, n=2, global_idx=[0, 1, 1], offsets=[0, 3, 3]), 1),
])
def test_create_rejects_bad_parameters(lib, kw, code):
    p, keep = _params(**kw)
    h = ctypes.c_void_p(1234)
    assert lib.swattn_create(ctypes.byref(p), ctypes.byref(h)) == code
    assert h.value == 1234  # untouched on failure
    assert lib.swattn_last_error().decode() != ""


def test_null_arguments(lib):
    h = ctypes.c_void_p()
    assert lib.swattn_create(None, ctypes.byref(h)) == 1
    p, keep = _params()
    assert lib.swattn_create(ctypes.byref(p), None) == 1
    assert lib.swattn_forward(None, *([None] * 9)) == 1
    assert lib.swattn_destroy(None) == 0


# swattn_project: every case below fails validation before any launch (the
# pointers are never dereferenced).
_X, _W, _O = 0x100000, 0x800000, 0x4000000


@pytest.mark.parametrize("args,code", [
    (dict(x=None), 1), (dict(w=None), 1), (dict(out=None), 1),
    (dict(batch=0), 1), (dict(n=0), 1), (dict(heads=0), 1), (dict(nproj=0), 1),
    (dict(d_model=0), 1),
    (dict(dtype=7), 2), (dict(d_model=80), 2),
    (dict(batch=1 << 20, n=1 << 10), 2),   # x of 2^30 * 64 * 2 bytes
    (dict(x=_X + 8), 4), (dict(bias=_W + 0x10000 + 8), 4), (dict(out=_O + 2), 4),
    (dict(out=_X + 64), 1),                # out overlaps x
])
def test_project_rejects_bad_parameters(lib, args, code):
    a = dict(x=_X, w=_W, bias=None, out=_O, batch=2, n=16, d_model=64, heads=2,
             nproj=3, dtype=0)
    a.update(args)
    lib.swattn_project.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int] * 6 + [ctypes.c_void_p]
    st = lib.swattn_project(a["x"], a["w"], a["bias"], a["out"], a["batch"], a["n"],
                            a["d_model"], a["heads"], a["nproj"], a["dtype"], None)
    assert st == code
    assert lib.swattn_last_error().decode() != ""
