"""Exact scaled-dot-product attention for MI355X (gfx950).

The compute path is a C-ABI shared library of hand-written HIP kernels
(``libattn.so``, built by ``__graft_entry__.build()``); ``binding`` is a thin
ctypes layer over it with the same entry-point names.  ``inputs`` draws the
seeded synthetic workloads; ``accounting`` counts their algorithmic work.

Importing the package does not load the library; the first call through
``binding`` does, and raises if the library is missing.
"""
