"""MXFP4 (E2M1 elements, one E8M0 scale per 32 along K) -- the plain definitions.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): never called by the
product path.

Sources, cited by page title and the part of the page:
  [517169] kernelbot amd-mxfp4-mm, submission 517169 -- module docstring (the
           "quantization math" list), ``_quant_to_fp4``, the sign/nibble packing
           inside ``_fused_quant_gemm_kernel``.
  [683203] kernelbot amd-mxfp4-mm, submission 683203 ("v3") -- docstring, trick 2
           (E8M0 byte 127 is the neutral scale 2^0); ``_quant_shuffled`` (block
           of 32 fixed by the OCP spec, M/K tail masks).
  [OCP-MX] OCP Microscaling Formats (MX) v1.0 specification -- E2M1 element
           encoding, E8M0 scale encoding, and the conversion rule
           shared_exp = floor(log2(amax)) - emax_elem with emax_elem = 2 for E2M1.

Readings taken where the pages are silent or disagree (each also listed in the
design notes): the scale rule is the OCP one, not the page-517169 docstring's
round(log2(amax/6)) nor its code's floor(log2(amax/6)); element rounding is
round-to-nearest with ties to the even code (the page-517169 threshold ladder
sends ties upward); the sign is bit 3 of the nibble (the page-517169 comment,
not its code, which ORs in 4); an all-zero block gets scale byte 127; the sign
of zero is kept (-0.0 encodes as 0x8); inputs must be finite.

Data conventions: bf16 tensors are carried as uint16 bit patterns (NumPy has no
bfloat16); packed fp4x2 and E8M0 scales are uint8.

Pins: every function here is checked in ``tests/test_oracle_pins.py`` against
values fixed by the pages and the mathematics (exhaustive decode, hand-worked
blocks, closed forms, invariants, exact rational brute force). The pages print
no numeric outputs of their own, so nothing is pinned to a page-printed result.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

# E2M1 magnitudes by 3-bit code 0..7 ([517169] docstring; [OCP-MX] FP4 table).
E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
# Largest power of two in E2M1 is 4 = 2^2 ([OCP-MX] emax for FP4 E2M1).
EMAX_E2M1 = 2
# Elements per shared scale ([683203] ``_quant_shuffled``: fixed at 32 by the OCP spec).
BLOCK = 32
# E8M0 stores the scale exponent with bias 127; byte 127 is 2^0 ([683203] trick 2).
SCALE_BIAS = 127
E8M0_MIN_EXP, E8M0_MAX_EXP = -127, 127  # byte 255 is NaN and is never produced

_GRID_FR = [Fraction(float(g)) for g in E2M1_GRID]  # exact binary fractions


# ----------------------------------------------------------------------------
# bf16 <-> float64
# ----------------------------------------------------------------------------
def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of each bf16 bit pattern (a bf16 is the top half of an fp32)."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 to bf16 (round to nearest, ties to even) and return the bits.

    bf16 keeps 8 significant bits with the fp32 exponent range: the quantum of a
    normal value x = m*2^e (m in [0.5,1)) is 2^(e-8); below 2^-126 the quantum is
    the subnormal step 2^-133. Results of magnitude 2^128 or more overflow to
    infinity. np.round rounds half to even.
    """
    x = np.asarray(x, dtype=np.float64)
    _, ex = np.frexp(x)
    q_exp = np.maximum(ex - 8, -133)
    y = np.ldexp(np.round(np.ldexp(x, -q_exp)), q_exp)
    y = np.where(np.abs(y) >= 2.0**128, np.copysign(np.inf, x), y)
    return (y.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# ----------------------------------------------------------------------------
# Quantisation (vectorised)
# ----------------------------------------------------------------------------
def shared_exponent(amax: np.ndarray) -> np.ndarray:
    """Per-block scale exponent e with scale 2^e ([OCP-MX] conversion rule).

    e = floor(log2(amax)) - EMAX_E2M1, clamped to the E8M0 range [-127, 127];
    a block whose amax is 0 gets e = 0 (scale 2^0). floor(log2) is read off the
    binary exponent (frexp gives amax = m*2^k with m in [0.5,1), so
    floor(log2 amax) = k-1), never from a floating-point log.
    """
    amax = np.asarray(amax, dtype=np.float64)
    _, k = np.frexp(amax)
    e = np.clip(k.astype(np.int64) - 1 - EMAX_E2M1, E8M0_MIN_EXP, E8M0_MAX_EXP)
    return np.where(amax == 0, 0, e).astype(np.int64)


def e2m1_code(m: np.ndarray) -> np.ndarray:
    """3-bit E2M1 code of magnitudes m >= 0: the nearest grid value, ties to the even code.

    "Nearest" covers saturation: every m >= 5 is nearest to 6 (code 7) except the
    tie m == 5, which goes to the even code 6 (value 4). The distances are exact
    in float64 for every m this is called with (m has at most 8 significant
    bits; when m is far below 0.25 a rounded distance still leaves code 0 the
    unique nearest), so the comparisons below are exact.
    """
    m = np.asarray(m, dtype=np.float64)
    d = np.abs(m[..., None] - E2M1_GRID)
    near = d == d.min(axis=-1, keepdims=True)
    lowest = np.argmax(near, axis=-1)  # smallest nearest code
    tie = near.sum(axis=-1) == 2       # two neighbours c, c+1 equally near
    # round half to even: of the tied pair keep the code whose low bit is 0
    return np.where(tie & (lowest % 2 == 1), lowest + 1, lowest).astype(np.uint8)


def quant_mx(x_bits: np.ndarray, rows_per_chunk: int = 256):
    """MXFP4 quantisation of a bf16 matrix X[R, K] along K.

    Returns (q, s): q uint8 [R, K/2] with element 2j in the low nibble and 2j+1
    in the high nibble of byte j ([517169] docstring and packing: low nibble =
    first); each nibble is sign (bit 3) | magnitude code (bits 0-2); s uint8
    [R, K/32], s = e + 127, block g covering k in [32g, 32g+32).

    Steps (per 32-element block): amax = max |x|; e = shared_exponent(amax);
    v = x / 2^e (exact); code = e2m1_code(|v|) | signbit(x) << 3.
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    if x_bits.ndim != 2:
        raise ValueError("quant_mx expects a 2-D [R, K] bf16 bit array")
    R, K = x_bits.shape
    if K % BLOCK != 0:
        raise ValueError(f"K={K} is not a multiple of {BLOCK}")
    q = np.empty((R, K // 2), dtype=np.uint8)
    s = np.empty((R, K // BLOCK), dtype=np.uint8)
    for r0 in range(0, R, rows_per_chunk):
        xb = x_bits[r0:r0 + rows_per_chunk]
        x = bf16_bits_to_f64(xb)
        if not np.all(np.isfinite(x)):
            raise ValueError("quant_mx: inputs must be finite")
        g = x.reshape(x.shape[0], K // BLOCK, BLOCK)
        amax = np.abs(g).max(axis=-1)
        e = shared_exponent(amax)
        v = np.ldexp(g, -e[..., None])
        mag = e2m1_code(np.abs(v)).reshape(x.shape[0], K)
        sign = (xb >> np.uint16(15)).astype(np.uint8)  # signbit, so -0.0 -> 1
        code = mag | (sign << np.uint8(3))
        q[r0:r0 + rows_per_chunk] = code[:, 0::2] | (code[:, 1::2] << np.uint8(4))
        s[r0:r0 + rows_per_chunk] = (e + SCALE_BIAS).astype(np.uint8)
    return q, s


def dequant_mx(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Values of packed MXFP4 data: (-1)^sign * E2M1[code & 7] * 2^(s - 127), float64 [R, K].

    copysign keeps the sign of a negative zero code (0x8 -> -0.0).
    """
    q = np.asarray(q, dtype=np.uint8)
    s = np.asarray(s, dtype=np.uint8)
    R, KH = q.shape
    K = 2 * KH
    if s.shape != (R, K // BLOCK):
        raise ValueError(f"scale shape {s.shape} does not match [{R}, {K // BLOCK}]")
    codes = np.empty((R, K), dtype=np.uint8)
    codes[:, 0::2] = q & np.uint8(0xF)
    codes[:, 1::2] = q >> np.uint8(4)
    mag = E2M1_GRID[codes & np.uint8(7)]
    val = np.copysign(mag, np.where(codes & np.uint8(8), -1.0, 1.0))
    exp = np.repeat(s.astype(np.int64) - SCALE_BIAS, BLOCK, axis=1)
    return np.ldexp(val, exp)


# ----------------------------------------------------------------------------
# GEMM
# ----------------------------------------------------------------------------
def gemm_ref_f64(a_bits: np.ndarray, bq: np.ndarray, bs: np.ndarray) -> np.ndarray:
    """C[m, n] = sum_k deq(Q(A))[m, k] * deq(B)[n, k] in float64 (B stored [N, K]).

    Orientation C = A B^T with B held as [N, K] follows every page
    ([517169] ``_fused_quant_gemm_kernel`` dots A against B transposed;
    [496271] kernelbot nvfp4-group-gemm, ``nvfp4_gemm_kernel`` the same).
    No alpha, beta or bias ([683203] passes alpha 1, beta 0, no bias).
    """
    aq, as_ = quant_mx(a_bits)
    return dequant_mx(aq, as_) @ dequant_mx(bq, bs).T


def gemm_ref(a_bits: np.ndarray, bq: np.ndarray, bs: np.ndarray) -> np.ndarray:
    """The fused op's reference output: gemm_ref_f64 rounded once to bf16 (bits, uint16)."""
    return f64_to_bf16_bits(gemm_ref_f64(a_bits, bq, bs))


# ----------------------------------------------------------------------------
# Scalar twins in exact arithmetic (for the small pin tests)
# ----------------------------------------------------------------------------
def _floor_log2(x: Fraction) -> int:
    k = x.numerator.bit_length() - x.denominator.bit_length()
    while Fraction(2) ** k > x:
        k -= 1
    while Fraction(2) ** (k + 1) <= x:
        k += 1
    return k


def quant_block_exact(xs):
    """One block of 32 finite floats -> (list of 32 nibble codes, scale byte), in exact rationals.

    Same definition as quant_mx, written independently over Fractions: the
    nearest E2M1 value to |x|/2^e, ties to the even code, sign from signbit.
    """
    if len(xs) != BLOCK:
        raise ValueError("a block has 32 elements")
    fr = [Fraction(float(x)) for x in xs]
    amax = max(abs(f) for f in fr)
    e = 0 if amax == 0 else max(E8M0_MIN_EXP, min(E8M0_MAX_EXP, _floor_log2(amax) - EMAX_E2M1))
    codes = []
    for x, f in zip(xs, fr):
        v = abs(f) / Fraction(2) ** e
        mag = min(range(8), key=lambda c: (abs(v - _GRID_FR[c]), c % 2))
        neg = math.copysign(1.0, float(x)) < 0
        codes.append((8 if neg else 0) | mag)
    return codes, e + SCALE_BIAS


def gemm_exact_fraction(a_vals, b_vals):
    """Exact rational C = A B^T for small lists of lists of Fractions (brute-force triple loop)."""
    M, K = len(a_vals), len(a_vals[0])
    N = len(b_vals)
    return [[sum((a_vals[m][k] * b_vals[n][k] for k in range(K)), Fraction(0)) for n in range(N)]
            for m in range(M)]
