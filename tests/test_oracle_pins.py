"""Pins of the CPU oracle against what the pages and the mathematics fix (no GPU).

Each test checks the oracle against something other than itself: the E2M1 table
and nibble/sign layout the pages state, hand-worked blocks (tests/golden), closed
forms computed from bf16 bit fields, an independent compare-ladder formulation of
round-to-nearest-even over every finite bf16 value, invariants of the OCP rule,
exact rational brute force for the GEMM, and an integer bf16 rounding. The
``test_planted_*`` tests plant a plausible mistake in the oracle and check that
the pins catch it.

Sources: kernelbot amd-mxfp4-mm submission 517169 (module docstring:
E2M1 grid, low nibble = first element; packing in ``_fused_quant_gemm_kernel``:
sign in bit 3), submission 683203 (docstring trick 2: byte 127 = 2^0), the OCP MX
v1.0 specification (shared exponent floor(log2 amax) - 2, E8M0 range).
"""
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import mx

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_blocks.txt")
E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def f32_bits(x):
    """bf16 bits of values that are exactly representable in bf16 (via fp32 truncation)."""
    b = np.asarray(x, dtype=np.float32).view(np.uint32)
    assert np.all((b & 0xFFFF) == 0), "value not representable in bf16"
    return (b >> 16).astype(np.uint16)


def block(head):
    return np.array(list(head) + [0.0] * (32 - len(head)), dtype=np.float64)


def ladder(m):
    """Independent RNE formulation: count midpoints passed, '>' at ties rounding down, '>=' up."""
    m = np.asarray(m, dtype=np.float64)
    return ((m > 0.25).astype(int) + (m >= 0.75) + (m > 1.25) + (m >= 1.75)
            + (m > 2.5) + (m >= 3.5) + (m > 5.0))


def scale_byte_from_bits(amax_bits):
    """Closed form from the bf16 exponent field: 127 for 0, else max(E - 2, 0)."""
    a = np.asarray(amax_bits, dtype=np.int64) & 0x7FFF
    return np.where(a == 0, 127, np.maximum((a >> 7) - 2, 0))


# ---------------------------------------------------------------------------
# decode / layout
# ---------------------------------------------------------------------------
def test_decode_all_16_codes():
    codes = np.arange(16, dtype=np.uint8)
    q = (codes[0::2] | (codes[1::2] << 4)).reshape(1, 8)
    q = np.concatenate([q, np.zeros((1, 8), np.uint8)], axis=1)  # one 32-element block
    v = oracle.dequant_mx(q, np.array([[127]], np.uint8))[0, :16]
    want = E2M1 + [-x for x in E2M1]
    assert v.tolist() == want
    assert not np.signbit(v[0]) and np.signbit(v[8])  # 0x8 decodes to -0.0


def test_nibble_order_and_sign_bit():
    x = block([0.5, -6.0])  # codes 0x1 and 0xF with scale 2^0
    q, s = oracle.quant_mx(f32_bits(x)[None])
    assert q[0, 0] == 0xF1 and s[0, 0] == 127
    assert q[0, 1:].tolist() == [0] * 15
    back = oracle.dequant_mx(q, s)[0]
    assert back[0] == 0.5 and back[1] == -6.0


def test_scale_applies_per_32_along_k():
    x = np.concatenate([block([1.0]), block([64.0])])
    q, s = oracle.quant_mx(f32_bits(x)[None])
    assert s.tolist() == [[125, 131]]


def _golden_rows():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            name, vals, sb, bts = [t.strip() for t in line.split("|")]
            vals = [float.fromhex(t) if t.startswith(("0x", "-0x")) else float(t) for t in vals.split()]
            rows.append((name, vals, int(sb), [int(t, 16) for t in bts.split()]))
    return rows


@pytest.mark.parametrize("name,vals,sbyte,lead", _golden_rows(), ids=[r[0] for r in _golden_rows()])
def test_hand_worked_blocks(name, vals, sbyte, lead):
    q, s = oracle.quant_mx(f32_bits(block(vals))[None])
    assert s[0, 0] == sbyte
    assert q[0, :len(lead)].tolist() == lead
    assert q[0, len(lead):].tolist() == [0] * (16 - len(lead))
    codes, sb2 = oracle.quant_block_exact(block(vals))
    assert sb2 == sbyte
    assert [codes[2 * j] | (codes[2 * j + 1] << 4) for j in range(len(lead))] == lead


@pytest.mark.parametrize("v,code", [(0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4), (3.5, 6), (5.0, 6)])
def test_ties_round_to_even_code(v, code):
    q, s = oracle.quant_mx(f32_bits(block([6.0, v]))[None])  # 6.0 pins the scale at 2^0
    assert s[0, 0] == 127
    assert (q[0, 0] >> 4) == code


@pytest.mark.parametrize("amax,byte", [(2.0**-126, 0), (2.0**-125, 0), (2.0**-124, 1), (1.0, 125),
                                       (6.0, 127), (2.0**100, 225), (2.0**-133, 0), (0.0, 127)])
def test_scale_byte_closed_form_points(amax, byte):
    _, s = oracle.quant_mx(f32_bits(block([amax]))[None])
    assert s[0, 0] == byte


def test_scale_byte_exhaustive_vs_exponent_field():
    bits = np.arange(0, 0x7F80, dtype=np.uint16)  # every non-negative finite bf16
    x = np.zeros((bits.size, 32), dtype=np.uint16)
    x[:, 5] = bits
    x[:, 9] = bits | 0x8000  # a negative copy must not change amax
    _, s = oracle.quant_mx(x)
    assert np.array_equal(s[:, 0].astype(np.int64), scale_byte_from_bits(bits))
    assert s.max() == 252  # bf16 max 0x7F7F -> E=254 -> 252; the upper clamp is unreachable


@pytest.mark.parametrize("anchor", [0.0, 2.0**-133, 2.0**-126, 2.0**-20, 1.0, 3.0, 7.5, 2.0**100, 1.5 * 2.0**127])
def test_every_bf16_element_code_vs_ladder(anchor):
    """Every finite bf16 x in a block with a fixed anchor: code == sign | ladder(|x| / 2^e)."""
    bits = np.arange(65536, dtype=np.uint32)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF].astype(np.uint16)  # finite only
    blk = np.zeros((bits.size, 32), dtype=np.uint16)
    blk[:, 0] = bits
    blk[:, 1] = f32_bits([anchor])[0]
    q, s = oracle.quant_mx(blk)
    xv = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    amax_bits = np.maximum(bits & 0x7FFF, f32_bits([anchor])[0])
    e = scale_byte_from_bits(amax_bits) - 127
    assert np.array_equal(s[:, 0].astype(np.int64), e + 127)
    want = ladder(np.abs(xv) * np.exp2(-e.astype(np.float64))) | ((bits >> 15).astype(int) << 3)
    assert np.array_equal((q[:, 0] & 0xF).astype(int), want)


# ---------------------------------------------------------------------------
# invariants on random blocks
# ---------------------------------------------------------------------------
def random_blocks(n, seed):
    g = np.random.default_rng(seed)
    x = g.standard_normal((n, 32)).astype(np.float32)
    x *= np.exp2(g.integers(-40, 40, size=(n, 1))).astype(np.float32)
    x[g.random((n, 32)) < 0.1] = 0.0
    x[: n // 50] *= np.float32(2.0**-100)  # some blocks deep in the clamped/subnormal range
    b = (x.view(np.uint32) >> 16).astype(np.uint16)  # truncation: any bf16 pattern is fine here
    b[n // 50: n // 25] = 0  # all-zero blocks
    return b


def test_invariants_random_blocks():
    b = random_blocks(10000, 1)
    q, s = oracle.quant_mx(b)
    x = oracle.bf16_bits_to_f64(b)
    e = s[:, 0].astype(np.int64) - 127
    d = oracle.dequant_mx(q, s)
    unclamped = (np.abs(x).max(1) > 0) & (e > -127)
    v = np.abs(x) * np.exp2(-e)[:, None]
    assert np.all(v[unclamped] < 8.0)
    assert np.all(np.abs(d) <= 6.0 * np.exp2(e)[:, None])
    codes = np.stack([q & 0xF, q >> 4], -1).reshape(q.shape[0], 32)
    top = (codes & 7).max(1)
    assert np.all(np.isin(top[unclamped], [6, 7]))
    # element error: half the local grid gap (at most 1 * 2^e), below 2 * 2^e when saturated
    err = np.abs(x - d) * np.exp2(-e)[:, None]
    sat = v > 6.0
    assert np.all(err[~sat] <= 1.0) and np.all(err[sat] < 2.0)
    # sign symmetry: negating flips bit 3 of every nibble and leaves the scale
    q2, s2 = oracle.quant_mx(b ^ np.uint16(0x8000))
    assert np.array_equal(q2, q ^ np.uint8(0x88)) and np.array_equal(s2, s)


def test_idempotent_on_dequantised_values():
    b = random_blocks(5000, 2)
    q, s = oracle.quant_mx(b)
    d = oracle.dequant_mx(q, s)
    back = f32_bits(d.astype(np.float32))
    q2, s2 = oracle.quant_mx(back)
    assert np.array_equal(q2, q)
    all_zero_mag = ((q & 0x77) == 0).all(1)  # blocks that dequantise to +-0 restart at scale 2^0
    assert np.array_equal(s2[~all_zero_mag], s[~all_zero_mag])
    assert np.all(s2[all_zero_mag] == 127)


def test_scale_equivariance():
    b = random_blocks(3000, 3)
    q, s = oracle.quant_mx(b)
    x = oracle.bf16_bits_to_f64(b)
    for j in (-3, 1, 5):
        ok = (s[:, 0].astype(int) + j > 0) & (s[:, 0].astype(int) + j < 253) & (np.abs(x).max(1) > 0)
        ok &= (s[:, 0] > 0)
        with np.errstate(under="ignore"):
            scaled = (x * 2.0**j).astype(np.float32)
        ok &= np.all(scaled.astype(np.float64) * 2.0**-j == x, axis=1)  # scaling stayed exact
        xs = f32_bits(scaled[ok])
        q2, s2 = oracle.quant_mx(xs)
        assert np.array_equal(q2, q[ok]) and np.array_equal(s2.astype(int), s[ok].astype(int) + j)


def test_vectorised_matches_exact_scalar_twin():
    b = random_blocks(400, 4)
    q, s = oracle.quant_mx(b)
    x = oracle.bf16_bits_to_f64(b)
    for r in range(b.shape[0]):
        codes, sb = oracle.quant_block_exact(x[r])
        assert sb == s[r, 0]
        assert [codes[2 * j] | (codes[2 * j + 1] << 4) for j in range(16)] == q[r].tolist()


# ---------------------------------------------------------------------------
# bf16 rounding of the output
# ---------------------------------------------------------------------------
def test_f64_to_bf16_halfway_cases():
    one = 1.0
    cases = [(one + 2.0**-8, 0x3F80), (one + 3 * 2.0**-8, 0x3F82), (-(one + 3 * 2.0**-8), 0xBF82),
             (1.0, 0x3F80), (2.0**-126, 0x0080), (2.0**-134, 0x0000), (3 * 2.0**-134, 0x0002),
             (2.0**-133, 0x0001), (2.0**128, 0x7F80), (0.0, 0x0000), (-0.0, 0x8000),
             ((2 - 2.0**-8) * 2.0**127, 0x7F80), ((2 - 2.0**-7) * 2.0**127, 0x7F7F)]
    for x, bits in cases:
        assert int(oracle.f64_to_bf16_bits(np.array([x]))[0]) == bits, x


def test_f64_to_bf16_vs_integer_rounding_of_fp32():
    g = np.random.default_rng(5)
    u = g.integers(0, 0x7F000000, size=200000, dtype=np.uint32)
    u |= (g.integers(0, 2, size=u.size, dtype=np.uint32) << 31)
    want = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    got = oracle.f64_to_bf16_bits(u.view(np.float32).astype(np.float64))
    assert np.array_equal(got, want)


# ---------------------------------------------------------------------------
# GEMM
# ---------------------------------------------------------------------------
def grid_exact_matrix(rows, K, g):
    """Values already on the MXFP4 grid with each block's max at 4*2^e or 6*2^e: quantisation is the identity."""
    codes = g.integers(0, 16, size=(rows, K))
    codes[:, ::32] = g.choice([6, 7, 14, 15], size=(rows, K // 32))
    mag = np.array(E2M1)[codes & 7]
    val = np.where(codes & 8, -mag, mag)
    e = g.integers(-10, 10, size=(rows, K // 32))
    return val * np.exp2(np.repeat(e, 32, axis=1))


def test_gemm_grid_exact_reduces_to_matmul():
    g = np.random.default_rng(6)
    A = grid_exact_matrix(8, 256, g)
    B = grid_exact_matrix(24, 256, g)
    Ab, Bb = f32_bits(A.astype(np.float32)), f32_bits(B.astype(np.float32))
    bq, bs = oracle.quant_mx(Bb)
    assert np.array_equal(oracle.dequant_mx(bq, bs), B)
    c = oracle.gemm_ref_f64(Ab, bq, bs)
    assert np.array_equal(c, A @ B.T)


def test_gemm_brute_force_fractions():
    g = np.random.default_rng(7)
    for M, N, K in [(1, 1, 32), (3, 5, 64), (8, 7, 128)]:
        a = f32_bits_round(g.standard_normal((M, K)) * np.exp2(g.integers(-3, 3, size=(M, 1))))
        b = f32_bits_round(g.standard_normal((N, K)) * 0.02)
        bq, bs = oracle.quant_mx(b)
        c64 = oracle.gemm_ref_f64(a, bq, bs)
        # exact: quantise each block with the rational twin, multiply with Fractions
        xa, xb = oracle.bf16_bits_to_f64(a), oracle.bf16_bits_to_f64(b)

        def exact_rows(x):
            out = []
            for r in range(x.shape[0]):
                row = []
                for kb in range(0, x.shape[1], 32):
                    codes, sb = oracle.quant_block_exact(x[r, kb:kb + 32])
                    for c in codes:
                        v = Fraction(E2M1[c & 7]) * Fraction(2) ** (sb - 127)
                        row.append(-v if c & 8 else v)
                out.append(row)
            return out

        exact = oracle.gemm_exact_fraction(exact_rows(xa), exact_rows(xb))
        assert np.array_equal(c64, np.array([[float(v) for v in r] for r in exact]))
        assert np.array_equal(oracle.gemm_ref(a, bq, bs),
                              oracle.f64_to_bf16_bits(np.array([[float(v) for v in r] for r in exact])))


def f32_bits_round(x):
    u = np.asarray(x, dtype=np.float32).view(np.uint32)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def test_gemm_orientation_is_a_times_b_transposed():
    a = f32_bits(block([1.0, 2.0])[None])                      # A[0, :2] = (1, 2)
    b = np.stack([f32_bits(block([4.0])), f32_bits(block([0.0, 4.0]))])  # rows of B[N=2, K]
    bq, bs = oracle.quant_mx(b)
    c = oracle.gemm_ref_f64(a, bq, bs)
    assert c.tolist() == [[4.0, 8.0]]  # C[0, n] = sum_k A[0,k] B[n,k]


def test_quant_rejects_bad_input():
    with pytest.raises(ValueError):
        oracle.quant_mx(np.zeros((2, 48), np.uint16))
    bad = np.zeros((1, 32), np.uint16)
    bad[0, 3] = 0x7F80  # +inf
    with pytest.raises(ValueError):
        oracle.quant_mx(bad)


# ---------------------------------------------------------------------------
# planted mistakes: each must be caught by the pins above
# ---------------------------------------------------------------------------
def _pins_pass():
    checks = [test_decode_all_16_codes, test_nibble_order_and_sign_bit, test_scale_applies_per_32_along_k,
              lambda: [test_hand_worked_blocks(*r) for r in _golden_rows()],
              lambda: [test_ties_round_to_even_code(v, c) for v, c in
                       [(0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4), (3.5, 6), (5.0, 6)]],
              test_scale_byte_exhaustive_vs_exponent_field,
              test_gemm_orientation_is_a_times_b_transposed]
    for c in checks:
        try:
            c()
        except AssertionError:
            return False
    return True


def test_pins_pass_unmodified():
    assert _pins_pass()


def test_planted_ties_upward_is_caught(monkeypatch):
    # the page-517169 ladder: strict thresholds, ties go up
    def up(m):
        m = np.asarray(m, dtype=np.float64)
        return sum((m >= t).astype(np.uint8) for t in (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)).astype(np.uint8)
    monkeypatch.setattr(mx, "e2m1_code", up)
    assert not _pins_pass()


def test_planted_sign_value_four_is_caught(monkeypatch):
    orig = mx.quant_mx

    def sign4(x_bits, rows_per_chunk=256):
        q, s = orig(np.asarray(x_bits, np.uint16) & np.uint16(0x7FFF))
        neg = (np.asarray(x_bits, np.uint16) >> 15).astype(np.uint8)
        return q | (neg[:, 0::2] << 2) | (neg[:, 1::2] << 6), s
    monkeypatch.setattr(mx, "quant_mx", sign4)
    monkeypatch.setattr(oracle, "quant_mx", sign4)
    assert not _pins_pass()


def test_planted_page_scale_rule_is_caught(monkeypatch):
    # floor(log2(amax / 6)) instead of floor(log2 amax) - 2
    def pagerule(amax):
        amax = np.asarray(amax, np.float64)
        with np.errstate(divide="ignore"):
            e = np.floor(np.log2(amax / 6.0 + 1e-30))
        return np.clip(e, -127, 127).astype(np.int64)
    monkeypatch.setattr(mx, "shared_exponent", pagerule)
    assert not _pins_pass()


def test_planted_swapped_nibbles_is_caught(monkeypatch):
    orig = mx.quant_mx

    def swapped(x_bits, rows_per_chunk=256):
        q, s = orig(x_bits)
        return ((q << 4) | (q >> 4)).astype(np.uint8), s
    monkeypatch.setattr(mx, "quant_mx", swapped)
    monkeypatch.setattr(oracle, "quant_mx", swapped)
    assert not _pins_pass()


def test_planted_b_read_as_k_by_n_is_caught(monkeypatch):
    # B taken as a [K, N] row-major matrix instead of [N, K]
    def wrong(a_bits, bq, bs):
        aq, as_ = mx.quant_mx(a_bits)
        A, B = mx.dequant_mx(aq, as_), mx.dequant_mx(bq, bs)
        return A @ B.reshape(B.shape[1], B.shape[0])
    monkeypatch.setattr(mx, "gemm_ref_f64", wrong)
    monkeypatch.setattr(oracle, "gemm_ref_f64", wrong)
    assert not _pins_pass()
