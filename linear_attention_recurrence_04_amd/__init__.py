"""Gated DeltaNet (gated delta rule) layer core for MI355X (gfx950).

The HIP library (``libgdn.so``) is loaded on first use by the binding, so the
seeded input generator can be imported on machines without a GPU.
"""
