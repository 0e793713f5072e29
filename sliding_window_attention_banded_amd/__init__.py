"""Banded sliding-window attention with global tokens for AMD MI355X (gfx950).

The compute path is the HIP library ``libswattn.so`` built from ``csrc/``;
``binding`` wraps its C ABI with ctypes (argument marshalling only). Importing
this package does not load the library; creating a ``Plan`` does, and fails
loudly when the library is missing.
"""

__all__ = ["Plan", "SwattnError", "project", "forward_noalloc", "library_path"]


def __getattr__(name):
    if name in __all__:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
