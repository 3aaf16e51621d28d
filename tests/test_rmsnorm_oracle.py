"""Pins of the RMSNorm + MXFP4 oracle (no GPU).

The pages name a kernel that fuses an RMSNorm with the MXFP4 quantisation
(kernelbot amd-mxfp4-mm submission 683203, docstring trick 1 and the comment
above ``_quant_shuffled``) but print none of its arithmetic, so these pins come
from the definition y = x / sqrt(mean(x^2) + eps) * w and from mathematics:
exact integer sums; the sum of squares equal to the exact rational sum rounded
once, on rows whose squares span many binades (where every fixed-order float64
sum loses bits); a closed form for constant rows; invariance under power-of-two
scaling of x; linearity in w; unit mean square; zero rows; and brute force over
a tiny row with Python's correctly rounded arithmetic. The ``test_planted_*``
tests plant plausible mistakes in the oracle and check that the pins catch them.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import mx, rmsnorm as rn


def bf16_bits(x):
    """bf16 bits (round to nearest even) of float64 values."""
    return mx.f64_to_bf16_bits(np.asarray(x, dtype=np.float64))


def rand_rows(rng, R, K, scale=1.0):
    return bf16_bits(rng.standard_normal((R, K)) * scale)


def test_sum_of_squares_exact_on_integers():
    rng = np.random.default_rng(1)
    x = rng.integers(-128, 129, size=(5, 7168)).astype(np.float64)  # bf16-exact integers
    ss = rn.rms_sum_squares(bf16_bits(x))
    assert np.array_equal(ss, (x.astype(np.int64) ** 2).sum(axis=1).astype(np.float64))


def exact_sum_squares(bits):
    """The exact rational sum of x^2 over a bf16 row, rounded once to float64 (Python's
    int / int division is correctly rounded)."""
    x = mx.bf16_bits_to_f64(bits)
    tot = sum(Fraction(float(v)) ** 2 for v in x)
    return tot.numerator / tot.denominator


def wide_rows(rng, K):
    """Rows whose squares span many binades, where any fixed-order float64 sum loses bits:
    one huge element among ones (2^54 + n with every +1 absorbed by naive summation), a
    row with exponents spread over +-40 binades, and one with tiny and huge values mixed."""
    big = np.ones(K)
    big[0] = 2.0**27
    spread = rng.standard_normal(K) * np.exp2(rng.integers(-40, 40, size=K))
    mixed = rng.standard_normal(K) * np.where(rng.random(K) < 0.01, 2.0**30, 2.0**-20)
    return [bf16_bits(big), bf16_bits(spread), bf16_bits(mixed)]


@pytest.mark.parametrize("K", [32, 96, 512, 1056, 7168])
def test_sum_of_squares_is_the_exact_sum_rounded_once(K):
    rng = np.random.default_rng(K)
    rows = [rand_rows(rng, 1, K)[0], rand_rows(rng, 1, K, 1e3)[0]] + wide_rows(rng, K)
    ss = rn.rms_sum_squares(np.stack(rows))
    for i, bits in enumerate(rows):
        assert ss[i] == exact_sum_squares(bits), (K, i)


def test_sum_of_squares_absorbs_nothing():
    """2^54 plus K-1 ones: the exact sum 2^54 + K - 1 is a float64 (K - 1 is a multiple of 4, the
    spacing at 2^54); a left-to-right float64 sum would stay at 2^54."""
    K = 7169
    x = np.ones((1, K))
    x[0, 0] = 2.0**27
    assert rn.rms_sum_squares(bf16_bits(x))[0] == 2.0**54 + (K - 1)


def test_constant_row_closed_form():
    K, eps = 7168, 2.0**-20
    for c in [1.0, -3.0, 0.15625, 96.0]:
        bits = bf16_bits(np.full((1, K), c))
        w = bf16_bits(np.ones(K))
        cb = float(mx.bf16_bits_to_f64(bits)[0, 0])
        inv = np.float32(1.0 / math.sqrt(cb * cb + eps))  # K*c^2/K is exact for these c
        want = bf16_bits(np.float64(np.float32(np.float32(cb) * inv)))
        y = rn.rmsnorm_bf16(bits, w, eps)
        assert np.all(y == want)


def test_power_of_two_invariance():
    rng = np.random.default_rng(7)
    x = rand_rows(rng, 6, 2048)
    w = rand_rows(rng, 1, 2048)[0]
    eps = 1e-30  # far below half an ulp of ss/K: the norm is then exactly scale-free
    y0 = rn.rmsnorm_bf16(x, w, eps)
    for k in [-12, -3, 1, 5, 17]:
        xk = bf16_bits(mx.bf16_bits_to_f64(x) * 2.0**k)
        assert np.array_equal(rn.rmsnorm_bf16(xk, w, eps), y0)


def test_linear_in_weight():
    rng = np.random.default_rng(8)
    x = rand_rows(rng, 4, 1024)
    w = rand_rows(rng, 1, 1024)[0]
    w2 = bf16_bits(mx.bf16_bits_to_f64(w) * 2.0)
    y = mx.bf16_bits_to_f64(rn.rmsnorm_bf16(x, w, 1e-6))
    y2 = mx.bf16_bits_to_f64(rn.rmsnorm_bf16(x, w2, 1e-6))
    assert np.array_equal(y2, 2.0 * y)


def test_unit_mean_square():
    rng = np.random.default_rng(9)
    x = rand_rows(rng, 8, 7168, 37.0)
    y = mx.bf16_bits_to_f64(rn.rmsnorm_bf16(x, bf16_bits(np.ones(7168)), 1e-12))
    assert np.all(np.abs((y * y).mean(axis=1) - 1.0) < 2.0**-6)


def test_zero_row_quantises_to_neutral_scale():
    x = np.zeros((2, 256), dtype=np.uint16)
    x[1, 5] = bf16_bits(np.array([2.0]))[0]
    q, s = rn.rmsnorm_quant(x, bf16_bits(np.ones(256)), 1e-6)
    assert np.all(q[0] == 0) and np.all(s[0] == 127)
    # row 1: one nonzero element of 2.0: ss = 4, inv = fp32(1/sqrt(4/256 + eps)) ~ 8, y = 16
    assert s[1, 0] == 127 + 2 and np.all(s[1, 1:] == 127)


def test_brute_force_tiny_row():
    """K = 64 row of small integers: every step by hand with Python floats."""
    rng = np.random.default_rng(10)
    K, eps = 64, 1e-5
    xi = rng.integers(-9, 10, size=K).astype(np.float64)
    wv = rng.standard_normal(K)
    x, w = bf16_bits(xi[None, :]), bf16_bits(wv)
    ss = float(sum(int(v) ** 2 for v in xi))  # exact, so any summation order agrees
    inv = np.float32(1.0 / math.sqrt(ss / K + float(np.float32(eps))))
    wf = mx.bf16_bits_to_f64(w)
    want = [bf16_bits(np.float64(np.float32(np.float32(np.float32(v) * inv) * np.float32(wk))))
            for v, wk in zip(xi, wf)]
    assert np.array_equal(rn.rmsnorm_bf16(x, w, eps)[0], np.array(want, dtype=np.uint16))
    q, s = rn.rmsnorm_quant(x, w, eps)
    q2, s2 = mx.quant_mx(np.array([want], dtype=np.uint16))
    assert np.array_equal(q, q2) and np.array_equal(s, s2)


def test_rejects_bad_eps():
    x = np.zeros((1, 32), dtype=np.uint16)
    for eps in [0.0, -1e-6, float("nan"), float("inf")]:
        with pytest.raises(ValueError):
            rn.rmsnorm_bf16(x, x[0], eps)


# -- planted mistakes: each must break at least one pin above --------------------------

def test_planted_fixed_order_sum_is_caught(monkeypatch):
    """A float64 sum in any fixed order (here left to right) is not the exact sum rounded once."""
    def naive(xb):
        x = mx.bf16_bits_to_f64(xb)
        out = np.zeros(x.shape[0])
        for k in range(x.shape[1]):
            out = out + x[:, k] * x[:, k]
        return out
    monkeypatch.setattr(rn, "rms_sum_squares", naive)
    with pytest.raises(AssertionError):
        test_sum_of_squares_absorbs_nothing()
    with pytest.raises(AssertionError):
        test_sum_of_squares_is_the_exact_sum_rounded_once(7168)


def test_planted_pairwise_sum_is_caught(monkeypatch):
    """numpy's pairwise summation is another fixed order: caught too."""
    monkeypatch.setattr(rn, "rms_sum_squares", lambda xb: (mx.bf16_bits_to_f64(xb) ** 2).sum(axis=1))
    with pytest.raises(AssertionError):
        test_sum_of_squares_is_the_exact_sum_rounded_once(7168)


def test_planted_missing_sqrt_is_caught(monkeypatch):
    monkeypatch.setattr(rn, "rms_inv", lambda ss, K, eps: (1.0 / (ss / K + eps)).astype(np.float32))
    with pytest.raises(AssertionError):
        test_power_of_two_invariance()


def test_planted_sum_of_abs_is_caught(monkeypatch):
    monkeypatch.setattr(rn, "rms_sum_squares", lambda xb: np.abs(mx.bf16_bits_to_f64(xb)).sum(axis=1))
    with pytest.raises(AssertionError):
        test_unit_mean_square()


def test_planted_mean_over_k_minus_one_is_caught(monkeypatch):
    monkeypatch.setattr(rn, "rms_inv", lambda ss, K, eps: (1.0 / np.sqrt(
        np.asarray(ss) / (K - 1) + np.float64(np.float32(eps)))).astype(np.float32))
    with pytest.raises(AssertionError):
        test_brute_force_tiny_row()
