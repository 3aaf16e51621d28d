"""NVFP4 (E2M1 elements, one E4M3 scale per 16 along K) block-scaled GEMM -- the plain definitions.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): never called by the
product path.

Sources, cited by page title and the part of the page:
  [496271] kernelbot nvfp4-group-gemm, submission 496271 -- module docstring
           (FP4 block scaling with the e2m1 element format on both operands),
           the constants block (one scale per 16 FP4 elements along K, two
           elements per byte), ``_prepare_scale_for_tma`` (the scales are
           float8_e4m3fn, one per (row, 16-element block) before reordering),
           ``nvfp4_gemm_kernel`` (C = A B^T with both operands held [rows, K/2],
           fp32 accumulation, the result stored as float16) and ``custom_kernel``
           (a list of problems, each with its own (m, n, k, l), l batches).
  [OCP-FP8] OCP 8-bit Floating Point Specification (OFP8) -- the E4M3 encoding:
           exponent bias 7, three mantissa bits, subnormals, no infinities,
           S.1111.111 is NaN, largest finite 448.
  [IEEE-754] binary16 -- 11 significant bits, exponents -14..15, subnormal
           quantum 2^-24, round to nearest even, overflow to infinity.

Readings taken where the page is silent (each also listed in the design notes):
the page shows no global (per-tensor) scale, so none is applied; E2M1 codes
use the same nibble order as the MXFP4 path (first element in the low nibble,
sign in bit 3); the scales are taken in their plain row-major [rows, K/16]
layout (the page reorders them for its tensor-memory loads, a layout of that
hardware); the output is float16 rounded once from the exact sum.

Pins: ``tests/test_nvfp4_oracle.py`` checks every function against the
library's own float8_e4m3fn and float16 conversions, hand-worked blocks,
exact rational brute force, invariants and a reduction to the MXFP4 oracle.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

from .mx import E2M1_GRID

# One E4M3 scale per 16 elements along K ([496271] constants block).
NV_BLOCK = 16
# E4M3 exponent bias and the NaN pattern S.1111.111 ([OCP-FP8]).
E4M3_BIAS = 7


def e4m3_to_f64(b: np.ndarray) -> np.ndarray:
    """Value of each E4M3 byte ([OCP-FP8]): (-1)^s * 2^(e-7) * (1 + m/8) for e > 0,
    (-1)^s * 2^-6 * m/8 for e = 0, NaN for the pattern with e = 15 and m = 7."""
    b = np.asarray(b, dtype=np.uint8).astype(np.int64)
    s = b >> 7
    e = (b >> 3) & 15
    m = b & 7
    mag = np.where(e > 0, np.ldexp(1.0 + m / 8.0, e - E4M3_BIAS), np.ldexp(m / 8.0, 1 - E4M3_BIAS))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


def e4m3_exact(b: int):
    """Exact Fraction value of one finite E4M3 byte (scalar twin of ``e4m3_to_f64``)."""
    s, e, m = b >> 7, (b >> 3) & 15, b & 7
    if e == 15 and m == 7:
        raise ValueError("E4M3 NaN")
    mag = Fraction(8 + m, 8) * Fraction(2) ** (e - E4M3_BIAS) if e else Fraction(m, 8) * Fraction(2) ** (1 - E4M3_BIAS)
    return -mag if s else mag


def f16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def f64_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 to binary16 (nearest, ties to even) and return the bits ([IEEE-754]).

    A normal x = f*2^e (f in [0.5, 1)) keeps 11 significant bits: quantum
    2^(e-11); below 2^-14 the quantum is the subnormal step 2^-24. Magnitudes
    that round to 2^16 or more overflow to infinity. np.round rounds half to even.
    """
    x = np.asarray(x, dtype=np.float64)
    _, ex = np.frexp(x)
    q_exp = np.maximum(ex - 11, -24)
    y = np.ldexp(np.round(np.ldexp(x, -q_exp)), q_exp)
    y = np.where(np.abs(y) >= 2.0**16, np.copysign(np.inf, x), y)
    y = np.where(np.isnan(x), np.nan, y)
    return y.astype(np.float16).view(np.uint16)  # y is already a binary16 value: the cast is exact


def nvfp4_dequant(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Values of NVFP4 data, float64 [R, K]: (-1)^sign * E2M1[code & 7] * E4M3(s[r, k // 16]).

    q: uint8 [R, K/2], element 2j in the low nibble of byte j, 2j+1 in the high
    nibble; s: uint8 E4M3 [R, K/16].
    """
    q = np.asarray(q, dtype=np.uint8)
    s = np.asarray(s, dtype=np.uint8)
    R, KH = q.shape
    K = 2 * KH
    if K % NV_BLOCK or s.shape != (R, K // NV_BLOCK):
        raise ValueError(f"scale shape {s.shape} does not match [{R}, {K // NV_BLOCK}]")
    codes = np.empty((R, K), dtype=np.uint8)
    codes[:, 0::2] = q & np.uint8(0xF)
    codes[:, 1::2] = q >> np.uint8(4)
    val = np.copysign(E2M1_GRID[codes & np.uint8(7)], np.where(codes & np.uint8(8), -1.0, 1.0))
    return val * np.repeat(e4m3_to_f64(s), NV_BLOCK, axis=1)


def nvfp4_gemm_f64(aq, as_, bq, bs) -> np.ndarray:
    """C[m, n] = sum_k deq(A)[m, k] * deq(B)[n, k] in float64, B held [N, K/2] ([496271]
    ``nvfp4_gemm_kernel``)."""
    return nvfp4_dequant(aq, as_) @ nvfp4_dequant(bq, bs).T


def nvfp4_gemm_ref(aq, as_, bq, bs) -> np.ndarray:
    """The reference output: ``nvfp4_gemm_f64`` rounded once to float16 (bits, uint16)."""
    return f64_to_f16_bits(nvfp4_gemm_f64(aq, as_, bq, bs))


def nvfp4_values_exact(q_row, s_row):
    """Exact Fractions of one row of NVFP4 data (scalar loop, for brute-force pins)."""
    out = []
    for k in range(2 * len(q_row)):
        byte = int(q_row[k // 2])
        code = byte & 15 if k % 2 == 0 else byte >> 4
        mag = Fraction(float(E2M1_GRID[code & 7]))
        out.append((-mag if code & 8 else mag) * e4m3_exact(int(s_row[k // NV_BLOCK])))
    return out
