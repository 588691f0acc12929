"""Fourier-approximated KV-cache decode on MI355X (gfx950).

The compute path is the C-ABI library ``libfa.so`` (hand-written HIP kernels,
sources under ``csrc/``); ``binding`` is a thin ctypes layer over it that takes
torch tensors for device memory and streams.  ``workloads`` draws seeded
synthetic inputs.  Importing this package does not load the library; the
binding loads it on first use and raises if it is missing.
"""
import importlib

__all__ = ["binding", "workloads"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module("." + name, __name__)
    raise AttributeError(name)
