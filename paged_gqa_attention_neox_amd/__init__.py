"""Paged GQA attention with NeoX rotary embedding for one MI355X (gfx950).

The compute lives in a C-ABI shared library of hand-written HIP kernels
(``libqwen2attn.so``, built from ``csrc/``).  This package is a thin ctypes
binding over it (``binding``) plus seeded synthetic inputs (``workloads``).
Importing the package loads nothing; the first binding call loads the
library and raises if it is missing.
"""
