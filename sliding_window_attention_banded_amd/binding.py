"""ctypes binding of libswattn.so (argument marshalling only).

Every step of the forward and backward passes runs in the HIP library; this module checks
tensor shapes and dtypes, hands raw device pointers and the current HIP
stream to the C ABI, and turns status codes into exceptions. PyTorch is used
for device memory and streams only. There is no fallback: if the library is
missing, creating a Plan raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["Plan", "SwattnError", "project", "forward_noalloc", "library_path", "load_library",
           "EXPORTS"]

_HERE = os.path.dirname(os.path.abspath(__file__))
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_HIP, ERR_ALIGNMENT = range(5)
BF16, FP32 = 0, 1
EXPORTS = ("swattn_create", "swattn_forward", "swattn_forward_noalloc", "swattn_backward",
           "swattn_project", "swattn_destroy",
           "swattn_set_timing", "swattn_kernel_times",
           "swattn_status_string", "swattn_last_error")


class SwattnError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{message} (status {status})")
        self.status = status


class _Params(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("n", ctypes.c_int32), ("d", ctypes.c_int32),
                ("window", ctypes.POINTER(ctypes.c_int32)),
                ("dilation", ctypes.POINTER(ctypes.c_int32)),
                ("causal", ctypes.c_int32),
                ("global_idx", ctypes.POINTER(ctypes.c_int32)),
                ("n_global", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("global_offsets", ctypes.POINTER(ctypes.c_int32)),
                ("key_split", ctypes.c_int32)]


def library_path():
    return os.environ.get("SWATTN_LIB", os.path.join(_HERE, "libswattn.so"))


_lib = None


def load_library():
    """Load libswattn.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise SwattnError(ERR_HIP, f"{path} is missing: build it with "
                          "`python -m sliding_window_attention_banded_amd.build`")
    lib = ctypes.CDLL(path)
    vp = ctypes.c_void_p
    lib.swattn_create.argtypes = [ctypes.POINTER(_Params), ctypes.POINTER(vp)]
    lib.swattn_create.restype = ctypes.c_int
    lib.swattn_forward.argtypes = [vp] * 8 + [vp, vp]
    lib.swattn_forward.restype = ctypes.c_int
    lib.swattn_forward_noalloc.argtypes = [ctypes.POINTER(_Params)] + [vp] * 9
    lib.swattn_forward_noalloc.restype = ctypes.c_int
    lib.swattn_backward.argtypes = [vp] * 17
    lib.swattn_backward.restype = ctypes.c_int
    lib.swattn_project.argtypes = [vp] * 4 + [ctypes.c_int] * 6 + [vp]
    lib.swattn_project.restype = ctypes.c_int
    lib.swattn_destroy.argtypes = [vp]
    lib.swattn_destroy.restype = ctypes.c_int
    lib.swattn_set_timing.argtypes = [vp, ctypes.c_int]
    lib.swattn_set_timing.restype = ctypes.c_int
    fp = ctypes.POINTER(ctypes.c_float)
    lib.swattn_kernel_times.argtypes = [vp, fp, fp, ctypes.POINTER(ctypes.c_int)]
    lib.swattn_kernel_times.restype = ctypes.c_int
    lib.swattn_status_string.argtypes = [ctypes.c_int]
    lib.swattn_status_string.restype = ctypes.c_char_p
    lib.swattn_last_error.argtypes = []
    lib.swattn_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(lib, status, what):
    if status != OK:
        name = lib.swattn_status_string(status).decode()
        msg = lib.swattn_last_error().decode()
        raise SwattnError(status, f"{what}: {name}: {msg}")


_DT = {torch.bfloat16: BF16, torch.float32: FP32}


class _ParamSet:
    """swattn_params for one configuration, with the host arrays it points
    to kept alive as long as this object."""

    def __init__(self, batch, heads, n, d, window, dilation, causal, global_idx, dtype,
                 key_split):
        if dtype not in _DT:
            raise SwattnError(ERR_UNSUPPORTED, f"dtype {dtype} not supported")
        win = [int(window)] * heads if isinstance(window, int) else [int(x) for x in window]
        dil = [int(dilation)] * heads if isinstance(dilation, int) else [int(x) for x in dilation]
        if len(win) != heads or len(dil) != heads:
            raise SwattnError(ERR_INVALID_ARG, "window/dilation need one entry per head")
        items = list(global_idx)
        per_item = bool(items) and all(isinstance(x, (list, tuple)) for x in items)
        if per_item:
            if len(items) != batch:
                raise SwattnError(ERR_INVALID_ARG, "per-example global_idx needs one list per batch item")
            sets = [[int(x) for x in g] for g in items]
            gl = [x for g in sets for x in g]
            offs = [0]
            for g in sets:
                offs.append(offs[-1] + len(g))
            self.global_idx = tuple(tuple(g) for g in sets)
        else:
            gl = [int(x) for x in items]
            offs = None
            self.global_idx = tuple(gl)
        self.has_globals = bool(gl)
        self.window, self.dilation = tuple(win), tuple(dil)
        self._W = (ctypes.c_int32 * heads)(*win)
        self._D = (ctypes.c_int32 * heads)(*dil)
        self._G = (ctypes.c_int32 * max(1, len(gl)))(*gl) if gl else None
        self._O = (ctypes.c_int32 * len(offs))(*offs) if offs else None
        self.params = _Params(batch, heads, n, d, self._W, self._D, int(bool(causal)),
                              ctypes.cast(self._G, ctypes.POINTER(ctypes.c_int32)) if self._G else None,
                              len(gl), _DT[dtype],
                              ctypes.cast(self._O, ctypes.POINTER(ctypes.c_int32)) if self._O else None,
                              int(key_split))


def _check_lse(lse, shape, device):
    if lse is None:
        return None
    if not lse.is_cuda or lse.device != device:
        raise SwattnError(ERR_INVALID_ARG, "lse must be a device tensor on the inputs' device")
    if lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != shape:
        raise SwattnError(ERR_INVALID_ARG, "lse must be contiguous fp32 [B, H, n]")
    return lse.data_ptr()


class Plan:
    """A configured banded-attention forward: ``Plan(...).forward(q, k, v)``.

    ``window`` and ``dilation`` are per head (a scalar is broadcast);
    ``global_idx`` lists the global-token positions shared by all batch items
    and heads, or gives one such list per batch item. Tensors are
    [B, H, n, 64] contiguous CUDA tensors in ``dtype``. ``key_split``: 0 lets
    the library share the band keys over several workgroups when the problem
    is too small to fill the GPU; 1 never does; k >= 2 always uses k parts.
    """

    def __init__(self, batch, heads, n, d=64, window=512, dilation=1,
                 causal=False, global_idx=(), dtype=torch.bfloat16, key_split=0):
        self._lib = load_library()
        ps = _ParamSet(batch, heads, n, d, window, dilation, causal, global_idx, dtype, key_split)
        self.global_idx = ps.global_idx
        self.has_globals = ps.has_globals
        self.batch, self.heads, self.n, self.d = batch, heads, n, d
        self.window, self.dilation, self.causal = ps.window, ps.dilation, bool(causal)
        self.dtype = dtype
        p = ps.params
        h = ctypes.c_void_p()
        _check(self._lib, self._lib.swattn_create(ctypes.byref(p), ctypes.byref(h)),
               "swattn_create")
        self._h = h

    def _ptr(self, t, name):
        if t is None:
            return None
        shape = (self.batch, self.heads, self.n, self.d)
        if not t.is_cuda:
            raise SwattnError(ERR_INVALID_ARG, f"{name} must be a device tensor")
        if t.dtype != self.dtype or tuple(t.shape) != shape or not t.is_contiguous():
            raise SwattnError(ERR_INVALID_ARG,
                              f"{name} must be contiguous {self.dtype} of shape {shape}")
        return t.data_ptr()

    def forward(self, q, k, v, qg=None, kg=None, vg=None, out=None, lse=None,
                want_lse=False, stream=None):
        """Enqueue one forward on the current stream; returns (out, lse)."""
        if self._h is None:
            raise SwattnError(ERR_INVALID_ARG, "plan is closed")
        if out is None:
            out = torch.empty_like(q)
        if lse is None and want_lse:
            lse = torch.empty((self.batch, self.heads, self.n), dtype=torch.float32,
                              device=q.device)
        lp = _check_lse(lse, (self.batch, self.heads, self.n), q.device)
        ptrs = [self._ptr(q, "q"), self._ptr(k, "k"), self._ptr(v, "v"),
                self._ptr(qg, "qg"), self._ptr(kg, "kg"), self._ptr(vg, "vg"),
                self._ptr(out, "out"), lp]
        st = stream if stream is not None else torch.cuda.current_stream(q.device)
        _check(self._lib, self._lib.swattn_forward(self._h, *ptrs, ctypes.c_void_p(st.cuda_stream)),
               "swattn_forward")
        return out, lse

    __call__ = forward

    def backward(self, q, k, v, o, lse, dout, qg=None, kg=None, vg=None,
                 grads=None, stream=None):
        """Enqueue the backward pass of a forward with these inputs and
        outputs (o, lse) for the cotangent ``dout``; returns the gradients
        (dq, dk, dv, dqg, dkg, dvg), the last three None without G.
        ``grads`` may supply the six output tensors."""
        if self._h is None:
            raise SwattnError(ERR_INVALID_ARG, "plan is closed")
        if lse is None:
            raise SwattnError(ERR_INVALID_ARG, "lse must be contiguous fp32 [B, H, n]")
        lp = _check_lse(lse, (self.batch, self.heads, self.n), q.device)
        has_g = self.has_globals
        if grads is None:
            grads = tuple(torch.empty_like(q) if (i < 3 or has_g) else None for i in range(6))
        names = ("dq", "dk", "dv", "dqg", "dkg", "dvg")
        gp = [self._ptr(t, nm) for t, nm in zip(grads, names)]
        ptrs = [self._ptr(q, "q"), self._ptr(k, "k"), self._ptr(v, "v"),
                self._ptr(qg, "qg"), self._ptr(kg, "kg"), self._ptr(vg, "vg"),
                self._ptr(o, "o"), lp, self._ptr(dout, "dout")] + gp
        st = stream if stream is not None else torch.cuda.current_stream(q.device)
        _check(self._lib, self._lib.swattn_backward(self._h, *ptrs, ctypes.c_void_p(st.cuda_stream)),
               "swattn_backward")
        return tuple(grads)

    def set_timing(self, enable=True):
        """Record HIP events around each kernel phase of later forwards."""
        _check(self._lib, self._lib.swattn_set_timing(self._h, int(bool(enable))),
               "swattn_set_timing")

    def kernel_times(self):
        """(band_ms, global_ms, count): average phase durations since the
        last call, measured with HIP events on the forward's stream."""
        b, g, c = ctypes.c_float(), ctypes.c_float(), ctypes.c_int()
        _check(self._lib, self._lib.swattn_kernel_times(self._h, ctypes.byref(b),
                                                        ctypes.byref(g), ctypes.byref(c)),
               "swattn_kernel_times")
        return b.value, g.value, c.value

    def close(self):
        if getattr(self, "_h", None) is not None:
            _check(self._lib, self._lib.swattn_destroy(self._h), "swattn_destroy")
            self._h = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def project(x, weight, bias=None, heads=None, out=None, stream=None):
    """Enqueue the projections in front of the attention (swattn_project):
    x [B, n, d_model], weight [P*heads*64, d_model] (a linear layer's
    layout), bias [P*heads*64] or None, all bf16 or all fp32. Returns out
    [P, B, heads, n, 64] of the same dtype; out[p] is projection p (q, k, v,
    then qg, kg, vg) in the layout Plan.forward takes."""
    lib = load_library()
    if heads is None or heads < 1:
        raise SwattnError(ERR_INVALID_ARG, "heads must be given and >= 1")
    dt = x.dtype
    if dt not in (torch.bfloat16, torch.float32):
        raise SwattnError(ERR_INVALID_ARG, "x must be bf16 or fp32")
    for name, t in (("x", x), ("weight", weight), ("bias", bias)):
        if t is None and name == "bias":
            continue
        if not t.is_cuda or t.dtype != dt or not t.is_contiguous():
            raise SwattnError(ERR_INVALID_ARG, f"{name} must be a contiguous {dt} device tensor like x")
    if x.dim() != 3 or weight.dim() != 2 or weight.shape[1] != x.shape[2] \
            or weight.shape[0] % (heads * 64) or weight.shape[0] == 0:
        raise SwattnError(ERR_INVALID_ARG, "need x [B, n, D] and weight [P*heads*64, D]")
    B, n, D = x.shape
    P = weight.shape[0] // (heads * 64)
    if bias is not None and tuple(bias.shape) != (P * heads * 64,):
        raise SwattnError(ERR_INVALID_ARG, "bias must be [P*heads*64]")
    shape = (P, B, heads, n, 64)
    if out is None:
        out = torch.empty(shape, dtype=dt, device=x.device)
    elif tuple(out.shape) != shape or out.dtype != dt or not out.is_contiguous() or not out.is_cuda:
        raise SwattnError(ERR_INVALID_ARG, f"out must be a contiguous {dt} device tensor of shape {shape}")
    st = stream if stream is not None else torch.cuda.current_stream(x.device)
    _check(lib, lib.swattn_project(x.data_ptr(), weight.data_ptr(),
                                   bias.data_ptr() if bias is not None else None,
                                   out.data_ptr(), B, n, D, heads, P,
                                   BF16 if dt == torch.bfloat16 else FP32,
                                   ctypes.c_void_p(st.cuda_stream)),
           "swattn_project")
    return out


def forward_noalloc(q, k, v, qg=None, kg=None, vg=None, window=512, dilation=1, causal=False,
                    global_idx=(), key_split=0, out=None, lse=None, want_lse=False, stream=None):
    """One forward through swattn_forward_noalloc: no plan, no device
    allocation inside the library (its tables and partial results live in a
    statically reserved device array shared by every call on the GPU, so
    calls must not overlap). Same arguments and result as
    ``Plan(...).forward``; the shape and dtype come from ``q``."""
    lib = load_library()
    if q.dim() != 4:
        raise SwattnError(ERR_INVALID_ARG, "q must be [B, H, n, d]")
    batch, heads, n, d = (int(x) for x in q.shape)
    ps = _ParamSet(batch, heads, n, d, window, dilation, causal, global_idx, q.dtype, key_split)
    shape = (batch, heads, n, d)

    def ptr(t, name):
        if t is None:
            return None
        if not t.is_cuda or t.device != q.device:
            raise SwattnError(ERR_INVALID_ARG, f"{name} must be a device tensor on q's device")
        if t.dtype != q.dtype or tuple(t.shape) != shape or not t.is_contiguous():
            raise SwattnError(ERR_INVALID_ARG, f"{name} must be contiguous {q.dtype} of shape {shape}")
        return t.data_ptr()

    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((batch, heads, n), dtype=torch.float32, device=q.device)
    lp = _check_lse(lse, (batch, heads, n), q.device)
    ptrs = [ptr(q, "q"), ptr(k, "k"), ptr(v, "v"), ptr(qg, "qg"), ptr(kg, "kg"), ptr(vg, "vg"),
            ptr(out, "out"), lp]
    st = stream if stream is not None else torch.cuda.current_stream(q.device)
    _check(lib, lib.swattn_forward_noalloc(ctypes.byref(ps.params), *ptrs,
                                           ctypes.c_void_p(st.cuda_stream)),
           "swattn_forward_noalloc")
    return out, lse
