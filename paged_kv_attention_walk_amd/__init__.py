"""Paged K/V split-K decode attention for MI355X (gfx950).

The compute path lives in the HIP library ``libpa_walk.so`` (C ABI declared in
``include/pa.h``); ``paged_kv_attention_walk_amd.binding`` is a thin ctypes
layer over it.  ``synth`` makes seeded synthetic inputs.  Importing this
package does not load the library; the first use of a binding name does, and
fails loudly when the library has not been built.
"""

import importlib

_SUBMODULES = ("binding", "synth", "build")


def __getattr__(name):
    if name in _SUBMODULES or name.startswith("_"):
        raise AttributeError(name)
    binding = importlib.import_module(__name__ + ".binding")
    try:
        return getattr(binding, name)
    except AttributeError:
        raise AttributeError(f"module {__name__!r} has no attribute {name!r}") from None
