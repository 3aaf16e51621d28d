"""Seeded sweep over problem shapes, on an MI355X: the fused call, gemm_a4w4 and
the grouped calls against the CPU oracle on random (M, N, K), so that every
kernel choice (split-K, the skinny kernel and its pre-quantised form, the
grouped kernel's skinny tiles with 1 to 4 sub-tiles and 64- or 128-column
tiles, the tiled kernel) meets M, N and K tails it was not hand-picked for.

C must satisfy |C - C_ref| <= 2^-7 |C_ref| + 1e-3 max|C_ref| elementwise (the
parity tests' bound); the fused call and gemm_a4w4 must agree bit for bit where
gemm_a4w4_fused_path says they run the same kernel. Shapes are drawn from one
fixed seed, sized so the oracle finishes each in about a second.
"""
import numpy as np
import pytest
import torch

import oracle
from mxfp4_block_scaled_02_amd import ops, synth
from tests.helpers import assert_in_tolerance, bits_of, to_dev_bf16, to_dev_u8

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


def _shapes(seed):
    """Six shapes from each of four ranges: M <= 16; 16 < M <= 64; a few hundred rows (where the skinny
    kernel or the grouped kernel's skinny tiles win); 600..1100 rows (mostly the tiled kernel)."""
    g = np.random.default_rng(seed)
    ranges = [((1, 17), (1, 4200), (1, 100)), ((17, 65), (1, 4200), (1, 100)), ((65, 521), (1000, 4200), (16, 129)),
              ((600, 1101), (2000, 4200), (8, 33))]
    out = []
    for (m0, m1), (n0, n1), (k0, k1) in ranges:
        got = 0
        while got < 6:
            M, N, K = int(g.integers(m0, m1)), int(g.integers(n0, n1)), 32 * int(g.integers(k0, k1))
            if M * N * K <= 1.5e9:
                out.append((M, N, K))
                got += 1
    return out


SINGLE = _shapes(2024)


def _operands(M, N, K, seed):
    g = np.random.default_rng(seed)
    a = synth.f32_to_bf16_bits((g.standard_normal((M, K)) * np.exp2(g.integers(-6, 6, (M, 1)))).astype(np.float32))
    b = synth.f32_to_bf16_bits((g.standard_normal((N, K)) * 0.02).astype(np.float32))
    return a, b


@pytest.mark.parametrize("M,N,K", SINGLE)
def test_fused_and_a4w4_random_shapes(M, N, K):
    path = ops.fused_path(M, N, K)
    say(f"sweep M={M} N={N} K={K} ({path})")
    a, b = _operands(M, N, K, M * 7 + N * 3 + K)
    bq, bs = oracle.quant_mx(b)
    at, bp = to_dev_bf16(a), ops.pack_B(to_dev_u8(bq), to_dev_u8(bs))
    cf = bits_of(ops.gemm(at, bp, N))
    aq, asc = ops.quant(at)
    c4 = bits_of(ops.gemm_a4w4(aq, asc, bp, N))
    ref = oracle.gemm_ref(a, bq, bs)
    assert_in_tolerance(cf, ref, f"fused M={M} N={N} K={K}")
    assert_in_tolerance(c4, ref, f"a4w4 M={M} N={N} K={K}")
    if (path == "splitk") if M <= 16 else (path in ("skinny", "tiled")):
        assert np.array_equal(c4, cf), f"fused and gemm_a4w4 differ on the same kernel ({path})"


def _group_lists(n, seed):
    g = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        G = int(g.integers(1, 7))
        Ms = [int(g.choice([g.integers(1, 65), g.integers(65, 513), g.integers(513, 900)], p=[0.5, 0.35, 0.15]))
              for _ in range(G)]
        N = int(g.integers(1, 3000))
        K = 32 * int(g.integers(1, 60))
        if sum(Ms) * N * K <= 6e8:
            out.append((Ms, N, K))
    return out


@pytest.mark.parametrize("Ms,N,K", _group_lists(10, 77))
def test_grouped_random_lists(Ms, N, K):
    say(f"sweep grouped Ms={Ms} N={N} K={K}")
    ops_ = [_operands(m, N, K, 1000 + i * 31 + m) for i, m in enumerate(Ms)]
    qs = [oracle.quant_mx(b) for _, b in ops_]
    cs = ops.grouped_gemm([to_dev_bf16(a) for a, _ in ops_], [ops.pack_B(to_dev_u8(q), to_dev_u8(s)) for q, s in qs], N)
    torch.cuda.synchronize()
    for (a, _), (bq, bs), c in zip(ops_, qs, cs):
        assert_in_tolerance(bits_of(c), oracle.gemm_ref(a, bq, bs), f"M={a.shape[0]} N={N} K={K}")


def _mnk_lists(n, seed):
    g = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        G = int(g.integers(1, 5))
        probs = []
        for _ in range(G):
            M = int(g.choice([g.integers(1, 65), g.integers(65, 513), g.integers(513, 800)], p=[0.45, 0.4, 0.15]))
            probs.append((M, int(g.integers(1, 2500)), 32 * int(g.integers(1, 48)), int(g.integers(1, 3))))
        if sum(M * N * K * L for M, N, K, L in probs) <= 8e8:
            out.append(probs)
    return out


@pytest.mark.parametrize("probs", _mnk_lists(8, 91))
def test_grouped_mnk_random_lists(probs):
    say(f"sweep grouped_mnk {probs}")
    groups = []
    for gi, (M, N, K, L) in enumerate(probs):
        pairs = [_operands(M, N, K, 5000 + 97 * gi + 13 * l) for l in range(L)]
        qs = [oracle.quant_mx(b) for _, b in pairs]
        A = torch.stack([to_dev_bf16(a) for a, _ in pairs])
        Bp = torch.stack([ops.pack_B(to_dev_u8(q), to_dev_u8(s)) for q, s in qs])
        groups.append(([a for a, _ in pairs], qs, A, Bp, N))
    outs = ops.grouped_gemm_mnk([(A, Bp, N) for _, _, A, Bp, N in groups])
    torch.cuda.synchronize()
    for (a_list, qs, _, _, N), C in zip(groups, outs):
        for l, (a, (bq, bs)) in enumerate(zip(a_list, qs)):
            assert_in_tolerance(bits_of(C[l]), oracle.gemm_ref(a, bq, bs), f"M={a.shape[0]} N={N} l={l}")


# Degenerate extents on every path: one column, a single K step (most waves of a skinny tile then own no
# K step and contribute zero partials), one to a few thousand rows.
EXTREMES = [(65, 1, 32), (512, 1, 32), (300, 5000, 32), (200, 4100, 32), (64, 1, 32), (1000, 1, 32), (129, 2, 64),
            (4096, 1, 32), (700, 130, 32), (17, 1, 32), (1, 1, 32), (2048, 4100, 32)]


@pytest.mark.parametrize("M,N,K", EXTREMES)
def test_extreme_extents(M, N, K):
    path = ops.fused_path(M, N, K)
    say(f"extreme M={M} N={N} K={K} ({path})")
    a, b = _operands(M, N, K, 3 * M + N + 7 * K)
    bq, bs = oracle.quant_mx(b)
    at, bp = to_dev_bf16(a), ops.pack_B(to_dev_u8(bq), to_dev_u8(bs))
    cf = bits_of(ops.gemm(at, bp, N))
    aq, asc = ops.quant(at)
    c4 = bits_of(ops.gemm_a4w4(aq, asc, bp, N))
    ref = oracle.gemm_ref(a, bq, bs)
    assert_in_tolerance(cf, ref, f"fused M={M} N={N} K={K}")
    assert_in_tolerance(c4, ref, f"a4w4 M={M} N={N} K={K}")


@pytest.mark.parametrize("Ms,N,K", [([100, 3, 300], 1, 32), ([64, 128], 2, 32), ([500, 40], 3000, 32), ([1, 1, 1], 1, 32)])
def test_grouped_extreme_extents(Ms, N, K):
    say(f"extreme grouped Ms={Ms} N={N} K={K}")
    ops_ = [_operands(m, N, K, 2000 + i * 17 + m) for i, m in enumerate(Ms)]
    qs = [oracle.quant_mx(b) for _, b in ops_]
    cs = ops.grouped_gemm([to_dev_bf16(a) for a, _ in ops_], [ops.pack_B(to_dev_u8(q), to_dev_u8(s)) for q, s in qs], N)
    torch.cuda.synchronize()
    for (a, _), (bq, bs), c in zip(ops_, qs, cs):
        assert_in_tolerance(bits_of(c), oracle.gemm_ref(a, bq, bs), f"M={a.shape[0]} N={N} K={K}")
