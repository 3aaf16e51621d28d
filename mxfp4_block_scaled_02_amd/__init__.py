"""Fused MXFP4 quantisation + block-scaled FP4 GEMM for MI355X (gfx950).

The compute lives in ``libmxfp4.so`` (hand-written HIP, C ABI declared in
``include/mxfp4.h``); ``ops`` marshals torch tensors into that ABI. Importing
this package does not load the library: ``ops`` loads it on first use and
raises if it is missing.
"""
__all__ = ["ops", "synth"]
