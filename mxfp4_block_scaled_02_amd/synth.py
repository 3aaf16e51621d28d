"""Seeded synthetic inputs for the fused MXFP4 quant + a4w4 GEMM.

This module draws random bf16 matrices and nothing else: it holds none of the
quantisation or GEMM arithmetic, so the CPU oracle and the HIP path can both be
fed from it without sharing any of the method's code. bf16 data are returned as
uint16 bit patterns (fp32 samples rounded to the nearest bf16, ties to even).

Workloads (the shapes the kernelbot amd-mxfp4-mm submissions work at: M=4 and
M=16 with K=7168 in the page-683203 / page-517169 docstrings, the M 4..256,
K 512..7168 regime of page 683203's launch policy, and the grouped form of the
kernelbot nvfp4-group-gemm submission 496271):

  tiny     M=4    N=256   K=512    A ~ N(0,1), B ~ N(0, 0.02)
  skinny   M=16   N=2112  K=7168   same distributions
  stress   M=64   N=7168  K=2048   A ~ N(0,1), exactly round(1% of M*K) distinct
                                   elements x50, then exactly round(2% of M*K/32)
                                   distinct 32-element groups set to +0.0;
                                   B ~ N(0,0.02) * 2^u per row, u ~ U[-8, 8]
  square   M=4096 N=4096  K=7168   A ~ N(0,1), B ~ N(0, 0.02)
  grouped  8 groups sharing N=4096, K=7168; M_g = 128 + 64*U{0..14};
           each group has its own A_g ~ N(0,1) and B_g ~ N(0,0.02)
  skinny_shard8  M=16 N=264 K7168: one GPU's share of skinny when N is split
           eight ways (skinny's A and the first 264 rows of its B, same seed)
  grouped_decode  the grouped form with decode-sized groups: 8 groups sharing
           N=4096, K=7168, M_g = 8*U{1..8} (each group's B read for a few rows,
           the case where a group of the list is HBM-bound)
  mid      M=256  N=4096  K=7168   the top of the M 4..256 regime; A ~ N(0,1),
                                   B ~ N(0, 0.02)

Every tensor draws from its own stream:
numpy PCG64(SeedSequence([seed, stream, *sub])). Streams: 0 = A, 1 = B,
2 = outlier/zero masks, 3 = B row exponents, 4 = group sizes.
"""
from __future__ import annotations

import numpy as np

WORKLOADS = {
    "tiny": dict(M=4, N=256, K=512),
    "skinny": dict(M=16, N=2112, K=7168),
    "stress": dict(M=64, N=7168, K=2048),
    "square": dict(M=4096, N=4096, K=7168),
    "grouped": dict(G=8, N=4096, K=7168),
    "skinny_shard8": dict(M=16, N=264, K=7168),
    "grouped_decode": dict(G=8, N=4096, K=7168),
    "mid": dict(M=256, N=4096, K=7168),
}
WORKLOAD_ORDER = ["tiny", "skinny", "stress", "square", "grouped", "grouped_decode", "mid"]
GROUPED = ("grouped", "grouped_decode")
SHARD_OF = {"skinny_shard8": "skinny"}  # a shard draws from its parent's seed

STREAM_A, STREAM_B, STREAM_MASK, STREAM_ROWEXP, STREAM_GROUPS, STREAM_NORM_W = 0, 1, 2, 3, 4, 5
STREAM_NV_CODES, STREAM_NV_SCALES = 6, 7


def rng(seed: int, stream: int, *sub: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream, *sub])))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Nearest bf16 (ties to even) of finite fp32 values, as uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def normal_bf16(shape, std: float, g: np.random.Generator) -> np.ndarray:
    x = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return f32_to_bf16_bits(x)


def make_a(M: int, K: int, seed: int, stream_sub=()) -> np.ndarray:
    return normal_bf16((M, K), 1.0, rng(seed, STREAM_A, *stream_sub))


def make_b(N: int, K: int, seed: int, stream_sub=()) -> np.ndarray:
    return normal_bf16((N, K), 0.02, rng(seed, STREAM_B, *stream_sub))


def make_norm_weight(K: int, seed: int) -> np.ndarray:
    """RMSNorm weight [K] as bf16 bits: 1 + N(0, 0.1), the usual shape of a trained norm gain."""
    w = np.float32(1.0) + np.float32(0.1) * rng(seed, STREAM_NORM_W).standard_normal(size=K, dtype=np.float32)
    return f32_to_bf16_bits(w)


def make_stress_a(M: int, K: int, seed: int) -> np.ndarray:
    x = rng(seed, STREAM_A).standard_normal(size=(M, K), dtype=np.float32)
    gm = rng(seed, STREAM_MASK)
    n_out = int(round(0.01 * M * K))
    pos = gm.choice(M * K, size=n_out, replace=False)
    x.reshape(-1)[pos] *= np.float32(50.0)
    n_groups = M * K // 32
    n_zero = int(round(0.02 * n_groups))
    grp = gm.choice(n_groups, size=n_zero, replace=False)
    x.reshape(n_groups, 32)[grp] = np.float32(0.0)
    return f32_to_bf16_bits(x)


def make_stress_b(N: int, K: int, seed: int) -> np.ndarray:
    x = rng(seed, STREAM_B).standard_normal(size=(N, K), dtype=np.float32) * np.float32(0.02)
    u = rng(seed, STREAM_ROWEXP).uniform(-8.0, 8.0, size=(N, 1))
    x *= np.exp2(u).astype(np.float32)
    return f32_to_bf16_bits(x)


def group_sizes(seed: int, G: int = 8) -> list:
    return [128 + 64 * int(v) for v in rng(seed, STREAM_GROUPS).integers(0, 15, size=G)]


def decode_group_sizes(seed: int, G: int = 8) -> list:
    return [8 * int(v) for v in rng(seed, STREAM_GROUPS).integers(1, 9, size=G)]


def workload(name: str, seed: int, rows=None):
    """Inputs of one workload: dict with M/N/K and bf16 bit arrays.

    ``rows`` (optional array of row indices) returns only those rows of A, drawn
    exactly as in the full tensor (the full A is generated, then sliced).
    For the grouped workloads the dict holds lists ``A`` and ``B`` and ``Ms``.
    """
    if name not in WORKLOADS:
        raise KeyError(name)
    w = dict(WORKLOADS[name])
    w["name"] = name
    w["seed"] = seed
    if name in GROUPED:
        Ms = (group_sizes if name == "grouped" else decode_group_sizes)(seed, w["G"])
        w["Ms"] = Ms
        w["A"] = [make_a(m, w["K"], seed, (g,)) for g, m in enumerate(Ms)]
        w["B"] = [make_b(w["N"], w["K"], seed, (g,)) for g in range(w["G"])]
        return w
    M, N, K = w["M"], w["N"], w["K"]
    if name == "stress":
        A, B = make_stress_a(M, K, seed), make_stress_b(N, K, seed)
    else:
        A, B = make_a(M, K, seed), make_b(N, K, seed)
    if rows is not None:
        A = A[np.asarray(rows)]
    w["A"], w["B"] = A, B
    return w


def default_seed(name: str) -> int:
    return WORKLOAD_ORDER.index(SHARD_OF.get(name, name))


def make_nvfp4(R: int, K: int, seed: int, stream_sub=()):
    """Random NVFP4 operand [R, K]: packed E2M1 codes uint8 [R, K/2], every byte
    uniform over 0..255 (all 16 codes equally likely, both signs), and E4M3
    scale bytes uint8 [R, K/16], positive, exponent field uniform in 4..10
    (2^-3 .. 2^3) and mantissa field uniform in 0..7. Raw bytes only."""
    codes = rng(seed, STREAM_NV_CODES, *stream_sub).integers(0, 256, size=(R, K // 2), dtype=np.uint8)
    g = rng(seed, STREAM_NV_SCALES, *stream_sub)
    e = g.integers(4, 11, size=(R, K // 16), dtype=np.uint8)
    m = g.integers(0, 8, size=(R, K // 16), dtype=np.uint8)
    return codes, ((e << np.uint8(3)) | m).astype(np.uint8)
