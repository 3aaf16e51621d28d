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
  - The sum of squares is taken in float64 in one fixed order, so that every
    implementation decides the quantised integers identically. Each x^2 is exact
    in float64. Lane t of 64 accumulates, in this order, its elements
    k = 512c + 8t + e (c = 0, 1, ...; e = 0..7; k < K). The 64 lane sums are then
    combined by a halving tree: S[t] += S[t + s] for s = 32, 16, 8, 4, 2, 1 and
    t < s. The sum is S[0].
  - inv = fp32(1 / sqrt(ss / K + eps)). Each float64 operation is correctly
    rounded, and so is the final conversion to fp32.
  - y_k = bf16(fp32(fp32(x_k * inv) * w_k)), each rounding to nearest, ties to
    even.
  - y is quantised by ``quant_mx``: an all-zero block (for example a zero row)
    gets scale byte 127.
"""
from __future__ import annotations

import numpy as np

from .mx import bf16_bits_to_f64, f64_to_bf16_bits, quant_mx

LANES = 64      # partial sums, one per lane of a 64-wide wave
CHUNK = 8       # consecutive elements a lane takes per pass
PASS = LANES * CHUNK  # 512 elements per pass over the row


def rms_sum_squares(x_bits: np.ndarray) -> np.ndarray:
    """Per-row sum of squares, float64, in the fixed order stated in the module docstring."""
    x = bf16_bits_to_f64(np.asarray(x_bits, dtype=np.uint16))
    if x.ndim != 2:
        raise ValueError("rms_sum_squares expects a 2-D [R, K] bf16 bit array")
    R, K = x.shape
    passes = -(-K // PASS)
    xx = np.zeros((R, passes * PASS), dtype=np.float64)
    xx[:, :K] = x * x  # exact; padding adds +0.0, which leaves every sum unchanged
    xx = xx.reshape(R, passes, LANES, CHUNK)
    lane = np.zeros((R, LANES), dtype=np.float64)
    for c in range(passes):          # lane order: pass by pass ...
        for e in range(CHUNK):       # ... and element by element within a pass
            lane = lane + xx[:, c, :, e]
    s = LANES // 2
    while s >= 1:                    # halving tree over the lanes
        lane[:, :s] = lane[:, :s] + lane[:, s:2 * s]
        s //= 2
    return lane[:, 0].copy()


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
