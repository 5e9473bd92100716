"""Flint routed-expert MoE layer for AMD MI355X (gfx950).

The compute runs in hand-written HIP kernels behind a C ABI
(include/flint_moe.h, libflint_moe.so); ``api`` is its Python binding and
``inputs`` draws the seeded synthetic workloads.  Importing the package does not
load the library; the first call through ``api`` does, and fails loudly if it is
missing.
"""
__all__ = ["api", "inputs"]
