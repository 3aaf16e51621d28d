"""Pins of the NVFP4 oracle (no GPU).

The NVFP4 page (kernelbot nvfp4-group-gemm, submission 496271) prints no
numbers of its own, so the pins come from the formats' definitions and from
mathematics: torch's own float8_e4m3fn decode and numpy's float16 rounding
(library routines independent of the oracle), hand-worked blocks, exact
rational brute force, the doubling invariant of a scale, and a reduction to
the MXFP4 oracle when every scale is 1. The ``test_planted_*`` tests plant
plausible mistakes in the oracle and check that a pin catches each.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import mx, nvfp4 as nv
from mxfp4_block_scaled_02_amd import synth


def test_e4m3_decode_matches_torch_for_all_256_codes():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = nv.e4m3_to_f64(np.arange(256))
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[~np.isnan(got)], ref[~np.isnan(ref)])
    assert np.array_equal(np.signbit(got), np.signbit(ref))  # 0x80 is -0


def test_e4m3_hand_values():
    assert nv.e4m3_to_f64(np.array([0x38]))[0] == 1.0  # e = 7, m = 0
    assert nv.e4m3_to_f64(np.array([0x7E]))[0] == 448.0  # the largest finite value
    assert nv.e4m3_to_f64(np.array([0x01]))[0] == 2.0**-9  # the smallest subnormal
    assert nv.e4m3_to_f64(np.array([0x08]))[0] == 2.0**-6  # the smallest normal
    assert nv.e4m3_to_f64(np.array([0x3D]))[0] == 1.625  # 1 + 5/8
    assert np.isnan(nv.e4m3_to_f64(np.array([0x7F, 0xFF]))).all()
    for b in range(256):
        if b & 0x7F != 0x7F:
            assert Fraction(float(nv.e4m3_to_f64(np.array([b]))[0])) == nv.e4m3_exact(b)


def test_f16_rounding_matches_numpy():
    g = np.random.default_rng(0)
    x = np.concatenate([
        g.standard_normal(20000) * np.exp2(g.integers(-30, 18, size=20000)),
        # exact ties: 11-bit significands plus half a quantum, normal and subnormal
        (np.arange(1, 4000, dtype=np.float64) * 2 + 1) * 2.0**-12,
        (np.arange(1, 2000, dtype=np.float64) * 2 + 1) * 2.0**-25,
        np.array([65504.0, 65519.0, 65520.0, 70000.0, -1e9, 2.0**-25, 2.0**-26, 0.0, -0.0]),
    ])
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(nv.f64_to_f16_bits(x), ref)


def test_dequant_hand_block():
    # one row, K = 32: codes 0..15 then 15..0; scales 2.0 (0x40) and 0.75 (0x34 = 2^-1 * 1.5)
    codes = list(range(16)) + list(range(15, -1, -1))
    q = np.array([[codes[2 * j] | (codes[2 * j + 1] << 4) for j in range(16)]], dtype=np.uint8)
    s = np.array([[0x40, 0x34]], dtype=np.uint8)
    grid = [0, .5, 1, 1.5, 2, 3, 4, 6]
    val = lambda c: (-1 if c & 8 else 1) * grid[c & 7]
    want = [val(c) * 2.0 for c in codes[:16]] + [val(c) * 0.75 for c in codes[16:]]
    got = nv.nvfp4_dequant(q, s)[0]
    assert np.array_equal(got, np.array(want))
    assert np.signbit(got[8]) and not np.signbit(got[0])  # code 8 is -0


def test_gemm_brute_force_exact():
    M, N, K = 3, 4, 48
    aq, as_ = synth.make_nvfp4(M, K, 11)
    bq, bs = synth.make_nvfp4(N, K, 12)
    as_[1, 2] = 0x01  # a subnormal scale
    bs[2, 0] = 0xB8  # a negative scale (-1)
    got = nv.nvfp4_gemm_f64(aq, as_, bq, bs)
    a = [nv.nvfp4_values_exact(aq[m], as_[m]) for m in range(M)]
    b = [nv.nvfp4_values_exact(bq[n], bs[n]) for n in range(N)]
    exact = mx.gemm_exact_fraction(a, b)
    for m in range(M):
        for n in range(N):
            assert Fraction(float(got[m, n])) == exact[m][n]  # short dyadic sums: float64 is exact here
    ref = nv.nvfp4_gemm_ref(aq, as_, bq, bs)
    want = np.array([[float(exact[m][n]) for n in range(N)] for m in range(M)]).astype(np.float16)
    assert np.array_equal(ref, want.view(np.uint16))


def test_scale_doubling_doubles_c():
    aq, as_ = synth.make_nvfp4(8, 256, 21)
    bq, bs = synth.make_nvfp4(16, 256, 22)
    c = nv.nvfp4_gemm_f64(aq, as_, bq, bs)
    as2 = (as_ + np.uint8(8)).astype(np.uint8)  # exponent field + 1 (fields are 4..10 here)
    assert np.array_equal(nv.nvfp4_gemm_f64(aq, as2, bq, bs), 2.0 * c)
    bs2 = bs.copy()
    bs2[:, 3] += np.uint8(8)  # one block of B doubled: only that block's products double
    d = nv.nvfp4_dequant(bq, bs)
    d[:, 48:64] *= 2.0
    assert np.allclose(nv.nvfp4_gemm_f64(aq, as_, bq, bs2), nv.nvfp4_dequant(aq, as_) @ d.T, rtol=0, atol=1e-9)


def test_unit_scales_reduce_to_mxfp4():
    """Every E4M3 scale 1.0 (0x38) is the MXFP4 GEMM with every E8M0 scale 2^0 (byte 127)."""
    aq, _ = synth.make_nvfp4(5, 128, 31)
    bq, _ = synth.make_nvfp4(7, 128, 32)
    one_nv = lambda r: np.full((r, 128 // 16), 0x38, dtype=np.uint8)
    one_mx = lambda r: np.full((r, 128 // 32), 127, dtype=np.uint8)
    c_nv = nv.nvfp4_gemm_f64(aq, one_nv(5), bq, one_nv(7))
    c_mx = mx.dequant_mx(aq, one_mx(5)) @ mx.dequant_mx(bq, one_mx(7)).T
    assert np.array_equal(c_nv, c_mx)


def test_rejects_bad_scale_shape():
    with pytest.raises(ValueError):
        nv.nvfp4_dequant(np.zeros((2, 16), np.uint8), np.zeros((2, 1), np.uint8))


# -- planted mistakes: each must break at least one pin above --------------------------

def test_planted_bias_8_is_caught(monkeypatch):
    monkeypatch.setattr(nv, "E4M3_BIAS", 8)
    with pytest.raises(AssertionError):
        test_e4m3_decode_matches_torch_for_all_256_codes()


def test_planted_block_of_32_is_caught(monkeypatch):
    monkeypatch.setattr(nv, "NV_BLOCK", 32)
    with pytest.raises((AssertionError, ValueError)):
        test_dequant_hand_block()


def test_planted_nibble_swap_is_caught(monkeypatch):
    real = nv.nvfp4_dequant

    def swapped(q, s):
        q = np.asarray(q, dtype=np.uint8)
        return real(((q >> 4) | (q << 4)).astype(np.uint8), s)

    monkeypatch.setattr(nv, "nvfp4_dequant", swapped)
    with pytest.raises(AssertionError):
        test_dequant_hand_block()


def test_planted_truncating_f16_is_caught(monkeypatch):
    def trunc(x):
        x = np.asarray(x, dtype=np.float64)
        _, ex = np.frexp(x)
        q = np.maximum(ex - 11, -24)
        with np.errstate(over="ignore"):
            return np.ldexp(np.trunc(np.ldexp(x, -q)), q).astype(np.float16).view(np.uint16)

    monkeypatch.setattr(nv, "f64_to_f16_bits", trunc)
    with pytest.raises(AssertionError):
        test_f16_rounding_matches_numpy()
