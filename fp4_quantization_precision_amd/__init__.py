"""libtq: block-scaled FP4 (NVFP4-style) quantization for MI355X (gfx950).

The compute lives in the HIP library libtq.so (C ABI in include/tq.h); the
``ops`` module is its torch binding and ``inputs`` draws the seeded synthetic
workloads.  Importing the package does not load the library; the first call
into ``ops`` does, and raises if it is not built.
"""
__all__ = ["ops", "inputs"]
