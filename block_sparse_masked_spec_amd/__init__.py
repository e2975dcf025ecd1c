"""Masked sparse attention (forward) for AMD MI355X (gfx950).

The compute path is the C-ABI library ``libsparse_attn.so`` built from
``csrc/`` (host planner + one fused HIP kernel).  ``binding`` is a thin
ctypes layer over it with the same function names.  Importing this package
loads nothing; ``from block_sparse_masked_spec_amd import binding`` loads the
library on first use, and ``inputs`` (the seeded generator) needs no build.
"""
