"""Paged-KV attention for MI355X (gfx950).

The compute path is a C-ABI shared library of hand-written HIP kernels
(csrc/); this package is its thin ctypes binding plus the seeded input
generators. Importing the package does not load the library; the first call
does, and raises if it has not been built.
"""
