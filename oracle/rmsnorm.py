"""RMSNorm followed by MXFP4 quantisation -- the plain definition.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): never called by the
product path.

Source: the pages name a kernel that fuses an RMSNorm with the MXFP4
quantisation (kernelbot amd-mxfp4-mm, submission 683203: docstring trick 1 and
the comment above ``_quant_shuffled``, whose scale-offset arithmetic comes from
it), but print none of its arithmetic. The norm here is the standard
root-mean-square layer normalisation, y = x / sqrt(mean(x^2) + eps) * w,
followed by the MXFP4 rule of ``oracle.mx.quant_mx``.

Readings taken because the pages are silent (each also listed in the design
notes):
  - w is a bf16 vector [K]; eps is an fp32 value > 0.
  - The sum of squares is the exact real sum of x_k^2 over the row, rounded
    once to float64 (nearest, ties to even). Each x_k^2 of a bf16 x_k is exact
    in float64 (8-bit significands), and math.fsum returns the correctly
    rounded sum of its float64 terms, so the result is independent of any
    summation order.
  - inv = fp32(1 / sqrt(ss / K + eps)). Each float64 operation is correctly
    rounded, and so is the final conversion to fp32.
  - y_k = bf16(fp32(fp32(x_k * inv) * w_k)), each rounding to nearest, ties to
    even.
  - y is quantised by ``quant_mx``: an all-zero block (for example a zero row)
    gets scale byte 127.
"""
from __future__ import annotations

import math

import numpy as np

from .mx import bf16_bits_to_f64, f64_to_bf16_bits, quant_mx


def rms_sum_squares(x_bits: np.ndarray) -> np.ndarray:
    """Per-row sum of x^2: the exact sum rounded once to float64."""
    x = bf16_bits_to_f64(np.asarray(x_bits, dtype=np.uint16))
    if x.ndim != 2:
        raise ValueError("rms_sum_squares expects a 2-D [R, K] bf16 bit array")
    sq = x * x  # exact: a bf16 square has at most 16 significant bits
    return np.array([math.fsum(row) for row in sq], dtype=np.float64)


def rms_inv(ss: np.ndarray, K: int, eps: float) -> np.ndarray:
    """fp32(1 / sqrt(ss / K + eps)) per row, each float64 step correctly rounded."""
    eps64 = np.float64(np.float32(eps))
    if not (np.isfinite(eps64) and eps64 > 0):
        raise ValueError("eps must be a finite fp32 value > 0")
    ms = np.asarray(ss, dtype=np.float64) / np.float64(K) + eps64
    return (np.float64(1.0) / np.sqrt(ms)).astype(np.float32)


def rmsnorm_bf16(x_bits: np.ndarray, w_bits: np.ndarray, eps: float) -> np.ndarray:
    """y = bf16(fp32(fp32(x * inv) * w)) as bf16 bits [R, K]."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    w_bits = np.asarray(w_bits, dtype=np.uint16).reshape(-1)
    R, K = x_bits.shape
    if w_bits.shape[0] != K:
        raise ValueError("w must have K elements")
    x = bf16_bits_to_f64(x_bits).astype(np.float32)  # exact: bf16 is a truncated fp32
    w = bf16_bits_to_f64(w_bits).astype(np.float32)
    if not (np.all(np.isfinite(x)) and np.all(np.isfinite(w))):
        raise ValueError("rmsnorm: inputs must be finite")
    inv = rms_inv(rms_sum_squares(x_bits), K, eps)
    with np.errstate(over="ignore"):
        t = x * inv[:, None]          # fp32 product, rounded to nearest even
        y = t * w[None, :]            # fp32 product, rounded to nearest even
    return f64_to_bf16_bits(y.astype(np.float64))


def rmsnorm_quant(x_bits: np.ndarray, w_bits: np.ndarray, eps: float):
    """(q, s) = quant_mx(rmsnorm_bf16(x, w, eps)): fp4x2 [R, K/2] and E8M0 [R, K/32]."""
    return quant_mx(rmsnorm_bf16(x_bits, w_bits, eps))
