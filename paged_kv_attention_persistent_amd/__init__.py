"""Paged decode attention in a persistent work-queue kernel, for MI355X (gfx950).

The product is the C-ABI shared library ``libpkv.so`` built from ``csrc/``
(its interface is ``include/pkv.h``).  ``pkv`` is the thin ctypes binding
with the same entry-point names; ``workloads`` makes seeded synthetic inputs.
Importing the package loads nothing; the library is loaded on first use and
a missing library is an error, never a fallback.
"""

__all__ = ["pkv", "workloads"]
