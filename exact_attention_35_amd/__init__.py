"""Exact attention (FlashAttention forward, backward, block-sparse forward) for MI355X / gfx950.

The compute lives in libfa.so (hand-written HIP kernels behind the C ABI of
include/fa.h); `api` marshals torch tensors into it.  `inputs` holds the
seeded synthetic workloads.  Importing the package does not load the library;
the first call does, and fails loudly if it has not been built.
"""

__all__ = ["api", "inputs", "build"]


def __getattr__(name):
    if name in ("api", "inputs", "build", "_lib"):
        import importlib

        return importlib.import_module(f".{name}", __name__)
    raise AttributeError(name)
