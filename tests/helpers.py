"""Shared test helpers: bf16 bit conversions and the C tolerance check."""
import numpy as np

import oracle


def to_dev_bf16(bits, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def to_dev_u8(a, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def bits_of(t):
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def tolerance_violations(c_bits, cref_bits):
    """|C - C_ref| <= 2^-7 |C_ref| + 1e-3 max|C_ref| elementwise (max over the given matrix)."""
    c = oracle.bf16_bits_to_f64(c_bits)
    r = oracle.bf16_bits_to_f64(cref_bits)
    tol = 2.0 ** -7 * np.abs(r) + 1e-3 * np.abs(r).max()
    bad = ~(np.abs(c - r) <= tol)
    return bad, c, r


def assert_in_tolerance(c_bits, cref_bits, what=""):
    bad, c, r = tolerance_violations(c_bits, cref_bits)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        detail = ", ".join(f"{tuple(i)}: got {c[tuple(i)]!r} want {r[tuple(i)]!r}" for i in idx)
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; first {detail}")


def quant_groups_in_pool(bs_list, workers=8):
    """Oracle-quantise several B matrices in spawned worker processes (CPU only)."""
    import concurrent.futures as cf
    import multiprocessing as mp
    ctx = mp.get_context("spawn")
    with cf.ProcessPoolExecutor(max_workers=min(workers, len(bs_list)), mp_context=ctx) as ex:
        return list(ex.map(oracle.quant_mx, bs_list))
