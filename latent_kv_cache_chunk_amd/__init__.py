"""Chunk-causal multi-head latent attention over a latent KV cache, for MI355X.

The compute path is a C-ABI shared library of hand-written HIP kernels for
gfx950 (``csrc/``, declared in ``include/mla.h``).  ``mla`` is the thin ctypes
binding over it: it marshals torch tensors (device memory and the current
stream) into plain pointers and raises ``MLAError`` on any non-OK status.
Importing the binding fails loudly when the built library is missing; there
is no CPU or PyTorch fallback.

``synth`` draws seeded synthetic workloads (no method arithmetic).
"""

import importlib

__all__ = ["mla", "synth"]


def __getattr__(name):
    # Lazy: importing the package (or .synth) must not need the built library.
    if name in __all__:
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
