"""Parity of grouped_gemm_a4w4_mnk (groups with their own M, N, K and a batch
count L, one launch; page 496271's problem form) with the CPU oracle, on an MI355X.

Each batch's C must be within |C - C_ref| <= 2^-7 |C_ref| + 1e-3 max|C_ref| of
the oracle's fp64 product of the dequantised operands rounded to bf16. Problems
with M > 64 run the tiled kernel, so where gemm_a4w4_fused runs it too
(gemm_a4w4_fused_path) the bytes must also equal the single-problem call's.
Problems of at most 64 rows take skinny tiles (K split over a workgroup's
waves) in the same launch.
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


def make_group(gi, M, N, K, L, seed):
    """L batches: bf16 bits of A [M, K] and B [N, K] per batch, plus device tensors."""
    a_bits = [synth.make_a(M, K, seed, (gi, l)) for l in range(L)]
    b_bits = [synth.make_b(N, K, seed, (gi, l)) for l in range(L)]
    bq = [oracle.quant_mx(b) for b in b_bits]
    A = torch.stack([to_dev_bf16(a) for a in a_bits])
    Bp = torch.stack([ops.pack_B(to_dev_u8(q), to_dev_u8(s)) for q, s in bq])
    return a_bits, bq, A, Bp


SHAPES = [(100, 300, 512, 2), (257, 1024, 2048, 1), (48, 96, 1056, 3), (130, 520, 7168, 1), (1, 32, 64, 2)]


def test_mixed_groups_match_oracle():
    say(f"[mnk] groups {SHAPES}")
    groups = [make_group(gi, M, N, K, L, 31) for gi, (M, N, K, L) in enumerate(SHAPES)]
    outs = ops.grouped_gemm_mnk([(A, Bp, N) for (_, _, A, Bp), (M, N, K, L) in zip(groups, SHAPES)])
    torch.cuda.synchronize()
    for (a_bits, bq, _, _), (M, N, K, L), C in zip(groups, SHAPES, outs):
        for l in range(L):
            assert_in_tolerance(bits_of(C[l]), oracle.gemm_ref(a_bits[l], *bq[l]), f"group M{M} N{N} K{K} l{l}")


def test_small_problems_beside_large_ones():
    """Problems of at most 64 rows take skinny tiles beside a large problem's tiled tiles, here of at most
    three 16-row sub-tiles (the fewest at which the launch fits one round of workgroups; the 64-row problem's
    second row tile has two sub-tiles past M): ragged N, a K tail on odd K/64, batches."""
    shapes = [(40, 4100, 1088, 3), (17, 2000, 832, 2), (600, 700, 1024, 1), (5, 4096, 512, 2), (48, 1000, 2048, 1), (64, 900, 704, 1)]
    say(f"[mnk] small and large {shapes}")
    groups = [make_group(gi, M, N, K, L, 35) for gi, (M, N, K, L) in enumerate(shapes)]
    outs = ops.grouped_gemm_mnk([(A, Bp, N) for (_, _, A, Bp), (M, N, K, L) in zip(groups, shapes)])
    torch.cuda.synchronize()
    for (a_bits, bq, _, _), (M, N, K, L), C in zip(groups, shapes, outs):
        for l in range(L):
            assert_in_tolerance(bits_of(C[l]), oracle.gemm_ref(a_bits[l], *bq[l]), f"group M{M} N{N} K{K} l{l}")


def test_mid_problems_on_skinny_tiles():
    """Problems of up to 512 rows take skinny tiles too when the launch model estimates the launch faster so
    (here every problem: a few hundred rows leave most CUs idle on 128 x 512 tiles); several row tiles per
    column, M tails, batches, odd K/64 tails."""
    shapes = [(130, 2048, 1056, 2), (300, 1000, 544, 1), (40, 512, 832, 1)]
    say(f"[mnk] mid problems {shapes}")
    groups = [make_group(gi, M, N, K, L, 38) for gi, (M, N, K, L) in enumerate(shapes)]
    outs = ops.grouped_gemm_mnk([(A, Bp, N) for (_, _, A, Bp), (M, N, K, L) in zip(groups, shapes)])
    torch.cuda.synchronize()
    for (a_bits, bq, _, _), (M, N, K, L), C in zip(groups, shapes, outs):
        for l in range(L):
            assert_in_tolerance(bits_of(C[l]), oracle.gemm_ref(a_bits[l], *bq[l]), f"group M{M} N{N} K{K} l{l}")


def test_small_problems_fewer_subtiles():
    """Small problems only, whose 16-row tiles would need a second round of workgroups: tiles of two 16-row
    sub-tiles, the 48-row problem's last one half past M; batches, odd K/64 tails."""
    shapes = [(48, 4096, 832, 2), (64, 2048, 704, 1), (17, 4096, 512, 1)]
    say(f"[mnk] capped sub-tiles {shapes}")
    groups = [make_group(gi, M, N, K, L, 37) for gi, (M, N, K, L) in enumerate(shapes)]
    outs = ops.grouped_gemm_mnk([(A, Bp, N) for (_, _, A, Bp), (M, N, K, L) in zip(groups, shapes)])
    torch.cuda.synchronize()
    for (a_bits, bq, _, _), (M, N, K, L), C in zip(groups, shapes, outs):
        for l in range(L):
            assert_in_tolerance(bits_of(C[l]), oracle.gemm_ref(a_bits[l], *bq[l]), f"group M{M} N{N} K{K} l{l}")


def test_large_m_groups_equal_single_calls():
    shapes = [(700, 4100, 1056, 1), (520, 4000, 704, 2), (1100, 2000, 1024, 1)]
    assert all(ops.fused_path(M, N, K) == "tiled" for M, N, K, _ in shapes)
    say(f"[mnk] vs single calls {shapes}")
    groups = [make_group(gi, M, N, K, L, 32) for gi, (M, N, K, L) in enumerate(shapes)]
    outs = ops.grouped_gemm_mnk([(A, Bp, N) for (_, _, A, Bp), (M, N, K, L) in zip(groups, shapes)])
    for (_, _, A, Bp), (M, N, K, L), C in zip(groups, shapes, outs):
        for l in range(L):
            single = ops.gemm(A[l], Bp[l], N)
            assert torch.equal(C[l].view(torch.int16), single.view(torch.int16)), (M, N, K, l)


def test_strided_batches():
    M, N, K, L = 70, 200, 1024, 3
    say(f"[mnk] strided batches M{M} N{N} K{K} L{L}")
    a_bits, bq, A, Bp = make_group(0, M, N, K, L, 33)
    Abig = torch.zeros((L, M + 5, K + 64), dtype=torch.bfloat16, device="cuda")
    Abig[:, :M, :K] = A
    Cbig = torch.full((L, M + 3, N + 24), float("nan"), dtype=torch.bfloat16, device="cuda")
    C = Cbig[:, :M, :N]
    ops.grouped_gemm_mnk([(Abig[:, :M, :K], Bp, N)], out_list=[C])
    torch.cuda.synchronize()
    for l in range(L):
        assert_in_tolerance(bits_of(C[l]), oracle.gemm_ref(a_bits[l], *bq[l]), f"l{l}")
    assert torch.isnan(Cbig[:, M:, :].float()).all() and torch.isnan(Cbig[:, :, N:].float()).all()


def test_thirty_two_problems():
    shapes = [(64 + 16 * g, 64 * (g % 3 + 1), 256 * (g % 2 + 1), 4) for g in range(8)]
    say("[mnk] 8 groups x 4 batches")
    groups = [make_group(gi, M, N, K, L, 34) for gi, (M, N, K, L) in enumerate(shapes)]
    outs = ops.grouped_gemm_mnk([(A, Bp, N) for (_, _, A, Bp), (M, N, K, L) in zip(groups, shapes)])
    torch.cuda.synchronize()
    for (a_bits, bq, _, _), (M, N, K, L), C in zip(groups, shapes, outs):
        for l in range(L):
            assert_in_tolerance(bits_of(C[l]), oracle.gemm_ref(a_bits[l], *bq[l]), f"M{M} N{N} K{K} l{l}")
