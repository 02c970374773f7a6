"""Decode-phase PagedAttention for MI355X (gfx950).

The compute lives in ``libpagedattn.so`` (hand-written HIP kernels behind a
C ABI, declared in ``include/pagedattn.h``); ``ops`` is a thin ctypes binding
over it. ``alloc`` (free-list block allocator), ``layouts`` (seeded synthetic
inputs) and ``sizing`` (byte counts) are host-side helpers.

Importing the package does not load the library; the first call into ``ops``
does, and fails loudly if it has not been built.
"""

__all__ = ["alloc", "layouts", "sizing", "ops"]


def __getattr__(name):
    if name in __all__:
        import importlib
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
