"""Argument checks of the Python binding that must stop a call before it
reaches the library (no kernel may see a host pointer): an LSE tensor that
is not on the inputs' device is rejected by Plan.forward, Plan.backward and
forward_noalloc."""
import pytest
import torch

from sliding_window_attention_banded_amd import binding


class _NoCall:
    """Stands in for the loaded library: any entry point reached fails."""

    def __getattr__(self, name):
        def fail(*a, **k):
            raise AssertionError(f"{name} was called")
        return fail


def _fake_plan(B=1, H=2, n=8):
    pl = object.__new__(binding.Plan)
    pl._lib = _NoCall()
    pl._h = object()
    pl.batch, pl.heads, pl.n, pl.d = B, H, n, 64
    pl.dtype = torch.bfloat16
    pl.has_globals = False
    return pl


def test_host_lse_is_rejected_before_the_library():
    pl = _fake_plan()
    q = torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16)
    lse = torch.zeros(1, 2, 8, dtype=torch.float32)
    with pytest.raises(binding.SwattnError, match="lse must be a device tensor"):
        pl.forward(q, q, q, lse=lse)
    with pytest.raises(binding.SwattnError, match="lse must be a device tensor"):
        pl.backward(q, q, q, q, lse, q)
    pl._h = None


@pytest.mark.gpu
def test_host_lse_with_device_inputs_is_rejected(monkeypatch):
    print("[binding] host lse with device inputs", flush=True)
    lib = binding.load_library()
    for name in ("swattn_forward", "swattn_backward", "swattn_forward_noalloc"):
        monkeypatch.setattr(lib, name, _NoCall().__getattr__(name))
    q = torch.zeros(1, 2, 256, 64, dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros(1, 2, 256, dtype=torch.float32)
    with binding.Plan(1, 2, 256, 64, 64, 1) as pl:
        with pytest.raises(binding.SwattnError, match="lse must be a device tensor"):
            pl.forward(q, q, q, lse=lse)
        with pytest.raises(binding.SwattnError, match="lse must be a device tensor"):
            pl.backward(q, q, q, q, lse, q)
    with pytest.raises(binding.SwattnError, match="lse must be a device tensor"):
        binding.forward_noalloc(q, q, q, window=64, lse=lse)
