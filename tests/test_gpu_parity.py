"""Parity of the HIP path (through the C ABI) with the CPU oracle, on an MI355X.

Quantised bytes (codes and E8M0 scales) must equal the oracle's bit for bit; C
must satisfy |C - C_ref| <= 2^-7 |C_ref| + 1e-3 max|C_ref| elementwise, C_ref the
oracle's fp64 product of the dequantised operands rounded once to bf16. Inputs
are the seeded synthetic workloads; B is always quantised by the oracle and
packed by mxfp4_pack_B. Large workloads run in the launch configuration the
benchmark times and are checked on sampled rows (the tolerance's max then runs
over the sample, which only tightens it).
"""
import numpy as np
import pytest
import torch

import oracle
from mxfp4_block_scaled_02_amd import ops, synth
from tests.helpers import (assert_in_tolerance, bits_of, quant_groups_in_pool, to_dev_bf16, to_dev_u8)

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


def gpu_quant(bits):
    q, s = ops.quant(to_dev_bf16(bits))
    return q.cpu().numpy(), s.cpu().numpy()


def packed_b(bq, bs):
    return ops.pack_B(to_dev_u8(bq), to_dev_u8(bs))


def run_gemm(a_bits, bq, bs, N, out=None):
    c = ops.gemm(to_dev_bf16(a_bits), packed_b(bq, bs), N, out=out)
    torch.cuda.synchronize()
    return c


# ---------------------------------------------------------------------------
# quantisation
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("anchor", [0.0, 2.0**-133, 2.0**-126, 1.0, 3.0, 7.5, 2.0**100, 1.5 * 2.0**127])
def test_quant_every_finite_bf16(anchor):
    say(f"quant exhaustive anchor={anchor!r}")
    bits = np.arange(65536, dtype=np.uint32)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF].astype(np.uint16)
    blk = np.zeros((bits.size, 32), dtype=np.uint16)
    blk[:, 0] = bits
    blk[:, 7] = (np.array([anchor], np.float32).view(np.uint32) >> 16).astype(np.uint16)[0]
    blk[:, 31] = bits[::-1]
    q, s = gpu_quant(blk)
    q0, s0 = oracle.quant_mx(blk)
    assert np.array_equal(s, s0)
    assert np.array_equal(q, q0)


@pytest.mark.parametrize("name", ["tiny", "skinny", "stress", "square"])
def test_quant_workload_bytes(name):
    say(f"quant workload {name}")
    w = synth.workload(name, synth.default_seed(name))
    for which in ("A", "B"):
        q, s = gpu_quant(w[which])
        q0, s0 = oracle.quant_mx(w[which])
        assert np.array_equal(s, s0), f"{name} {which} scales"
        assert np.array_equal(q, q0), f"{name} {which} codes"


@pytest.mark.timeout(600)
def test_quant_workload_bytes_grouped():
    say("quant workload grouped (every group's A and B)")
    w = synth.workload("grouped", synth.default_seed("grouped"))
    mats = list(w["A"]) + list(w["B"])
    refs = quant_groups_in_pool(mats)
    for i, (x, (q0, s0)) in enumerate(zip(mats, refs)):
        q, s = gpu_quant(x)
        what = f"grouped {'A' if i < len(w['A']) else 'B'}{i % len(w['A'])}"
        assert np.array_equal(s, s0), f"{what} scales"
        assert np.array_equal(q, q0), f"{what} codes"


@pytest.mark.parametrize("M,K", [(1, 32), (3, 96), (17, 32), (5, 7168), (300, 224)])
def test_quant_edge_shapes_and_strides(M, K):
    say(f"quant edge M={M} K={K}")
    g = np.random.default_rng(M * 1000 + K)
    x = synth.f32_to_bf16_bits((g.standard_normal((M, K)) * np.exp2(g.integers(-130, 120, (M, 1)))).astype(np.float32))
    x[0, :2] = [0x8000, 0x0001]  # -0.0 and the smallest subnormal
    if K >= 64:
        x[0, 32:64] = 0x8000  # an all -0.0 block
    x[-1, -1] = 0x7F7F  # bf16 max
    q0, s0 = oracle.quant_mx(x)
    # strided input and outputs inside larger buffers
    ldx, ldq, lds = K + 8, K // 2 + 16, K // 32 + 3
    xb = np.zeros((M, ldx), np.uint16)
    xb[:, :K] = x
    xt = to_dev_bf16(xb)
    qt = torch.full((M, ldq), 0xAB, dtype=torch.uint8, device="cuda")
    st = torch.full((M, lds), 0xCD, dtype=torch.uint8, device="cuda")
    rc = ops.lib().mxfp4_quant(xt.data_ptr(), ldx, qt.data_ptr(), ldq, st.data_ptr(), lds, M, K,
                               torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    qn, sn = qt.cpu().numpy(), st.cpu().numpy()
    assert np.array_equal(qn[:, :K // 2], q0) and np.array_equal(sn[:, :K // 32], s0)
    assert (qn[:, K // 2:] == 0xAB).all() and (sn[:, K // 32:] == 0xCD).all()  # guard bytes untouched


def test_quant_repeatable():
    w = synth.workload("stress", 2)
    runs = [gpu_quant(w["A"]) for _ in range(5)]
    for q, s in runs[1:]:
        assert np.array_equal(q, runs[0][0]) and np.array_equal(s, runs[0][1])


# ---------------------------------------------------------------------------
# packing of B
# ---------------------------------------------------------------------------
def host_pack(bq, bs):
    """The layout stated in include/mxfp4.h, written out with NumPy indexing."""
    N, KH = bq.shape
    K = 2 * KH
    NT, KU = -(-N // 32), -(-K // 64)
    KG = -(-KU // 4)
    Np, Kp = NT * 32, KU * 64
    codes = np.zeros((Np, Kp // 2), np.uint8)
    codes[:N, :K // 2] = bq
    # unit (t, u), lane l: row 32t + l%32, bytes (64u + 32(l/32))/2 .. +16
    units = codes.reshape(NT, 32, KU, 2, 16).transpose(0, 2, 3, 1, 4).reshape(-1)
    sc = np.full((Np, KG * 8), 127, np.uint8)
    sc[:N, :K // 32] = bs
    # dword (t, g, l): byte i = scale[32t + l%32, 2(4g+i) + l/32]
    scal = sc.reshape(NT, 32, KG, 4, 2).transpose(0, 2, 4, 1, 3).reshape(-1)
    return np.concatenate([units, scal])


@pytest.mark.parametrize("N,K", [(37, 352), (16, 128), (2112, 7168), (5, 32)])
def test_pack_B_layout(N, K):
    say(f"pack_B N={N} K={K}")
    g = np.random.default_rng(N + K)
    bq = g.integers(0, 256, (N, K // 2), dtype=np.uint8)
    bs = g.integers(100, 150, (N, K // 32), dtype=np.uint8)
    got = packed_b(bq, bs).cpu().numpy()
    assert np.array_equal(got, host_pack(bq, bs))


# ---------------------------------------------------------------------------
# fused GEMM
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["tiny", "skinny", "stress", "skinny_shard8", "mid"])
def test_gemm_workload_full(name):
    say(f"gemm workload {name}")
    w = synth.workload(name, synth.default_seed(name))
    bq, bs = oracle.quant_mx(w["B"])
    c = run_gemm(w["A"], bq, bs, w["N"])
    assert_in_tolerance(bits_of(c), oracle.gemm_ref(w["A"], bq, bs), name)


def test_gemm_square_sampled_rows():
    say("gemm workload square (sampled rows)")
    w = synth.workload("square", synth.default_seed("square"))
    bq, bs = oracle.quant_mx(w["B"])
    c = bits_of(run_gemm(w["A"], bq, bs, w["N"]))
    rows = np.unique(np.concatenate([np.arange(16), np.arange(4096 - 16, 4096),
                                     np.random.default_rng(0).choice(4096, 48, replace=False)]))
    assert_in_tolerance(c[rows], oracle.gemm_ref(w["A"][rows], bq, bs), "square")


# Robustness runs: the same workloads from a second seed (100 + the workload's index).
@pytest.mark.parametrize("name", ["tiny", "skinny", "stress"])
def test_workload_second_seed(name):
    seed = 100 + synth.default_seed(name)
    say(f"workload {name} seed {seed}: quant bytes and full C")
    w = synth.workload(name, seed)
    q, s = gpu_quant(w["A"])
    rq, rs = oracle.quant_mx(w["A"])
    assert np.array_equal(q, rq) and np.array_equal(s, rs)
    bq, bs = oracle.quant_mx(w["B"])
    c = run_gemm(w["A"], bq, bs, w["N"])
    assert_in_tolerance(bits_of(c), oracle.gemm_ref(w["A"], bq, bs), f"{name} seed {seed}")


def test_square_second_seed_sampled_rows():
    seed = 100 + synth.default_seed("square")
    say(f"gemm workload square seed {seed} (sampled rows)")
    w = synth.workload("square", seed)
    bq, bs = oracle.quant_mx(w["B"])
    c = bits_of(run_gemm(w["A"], bq, bs, w["N"]))
    rows = np.unique(np.concatenate([np.arange(8), np.arange(4096 - 8, 4096),
                                     np.random.default_rng(seed).choice(4096, 32, replace=False)]))
    assert_in_tolerance(c[rows], oracle.gemm_ref(w["A"][rows], bq, bs), f"square seed {seed}")


@pytest.mark.timeout(600)
def test_grouped_workload_sampled_rows():
    say("grouped workload (sampled rows)")
    w = synth.workload("grouped", synth.default_seed("grouped"))
    qs = quant_groups_in_pool(w["B"])
    a_dev = [to_dev_bf16(a) for a in w["A"]]
    bp = [packed_b(bq, bs) for bq, bs in qs]
    cs = ops.grouped_gemm(a_dev, bp, w["N"])
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    for g, (a, (bq, bs), c) in enumerate(zip(w["A"], qs, cs)):
        m = a.shape[0]
        rows = np.unique(np.concatenate([[0, m - 1], rng.choice(m, 14, replace=False)]))
        assert_in_tolerance(bits_of(c)[rows], oracle.gemm_ref(a[rows], bq, bs), f"group {g} (M={m})")


EDGE = [(1, 1, 32), (1, 16, 128), (2, 100, 96), (4, 256, 512), (16, 2112, 7168), (17, 50, 160), (33, 64, 352),
        (64, 130, 2048), (65, 130, 288), (127, 257, 1056), (255, 300, 4096), (1, 4096, 7168), (300, 33, 32),
        # split-K path (M <= 16): K tail with M < 16; odd K/64 with a K tail (9 splits of 6-7 steps);
        # the 64-split maximum; more K than 64 splits can hold (falls back to the skinny kernel); a
        # middle case; the 8-way N shard of skinny
        (3, 70, 352), (16, 130, 7232), (16, 64, 65536), (16, 48, 66560), (8, 1000, 6144), (16, 264, 7168),
        # M <= 16 where the skinny kernel (K split over one workgroup's waves, no hand-off) is estimated
        # faster than split-K: wide N, or a short K that split-K would cut into one-step splits
        (8, 4096, 7168), (16, 7168, 2048), (2, 4096, 4096), (16, 130, 1088), (5, 300, 1024),
        # 16 < M <= 64 on 128-column workgroups: an M tail, a ragged N, odd K/64 with a K tail
        (50, 20000, 1056)]


@pytest.mark.parametrize("M,N,K", EDGE)
def test_gemm_edge_shapes(M, N, K):
    say(f"gemm edge M={M} N={N} K={K}")
    g = np.random.default_rng(M * 7 + N * 13 + K)
    a = synth.f32_to_bf16_bits(g.standard_normal((M, K)).astype(np.float32))
    b = synth.f32_to_bf16_bits((g.standard_normal((N, K)) * 0.02).astype(np.float32))
    bq, bs = oracle.quant_mx(b)
    c = run_gemm(a, bq, bs, N)
    assert_in_tolerance(bits_of(c), oracle.gemm_ref(a, bq, bs), f"M={M} N={N} K={K}")


@pytest.mark.parametrize("M,N,K", [(16, 2112, 7168), (70, 200, 512)])
def test_gemm_strides_and_guard_band(M, N, K):
    say(f"gemm strided M={M} N={N} K={K}")
    g = np.random.default_rng(11)
    a = synth.f32_to_bf16_bits(g.standard_normal((M, K)).astype(np.float32))
    b = synth.f32_to_bf16_bits((g.standard_normal((N, K)) * 0.02).astype(np.float32))
    bq, bs = oracle.quant_mx(b)
    lda, ldc = K + 64, N + 24
    abuf = np.zeros((M, lda), np.uint16)
    abuf[:, :K] = a
    abuf[:, K:] = 0x7F7F  # garbage beyond K must be ignored
    at = to_dev_bf16(abuf)
    cbuf = torch.full((M + 2, ldc), 1234.0, dtype=torch.bfloat16, device="cuda")
    cview = cbuf[1:M + 1]
    bp = packed_b(bq, bs)
    wsz = ops.lib().gemm_a4w4_workspace_bytes(M, N, K)
    ws = ops.workspace(at.device, wsz)
    rc = ops.lib().gemm_a4w4_fused(at.data_ptr(), lda, bp.data_ptr(), cview.data_ptr(), ldc, M, N, K,
                                   ws.data_ptr() if wsz else None, ws.numel() if wsz else 0,
                                   torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    cb = bits_of(cbuf)
    assert_in_tolerance(cb[1:M + 1, :N], oracle.gemm_ref(a, bq, bs), "strided")
    guard = bits_of(torch.tensor([1234.0], dtype=torch.bfloat16))[0]
    assert (cb[0] == guard).all() and (cb[M + 1] == guard).all() and (cb[:, N:] == guard).all()


@pytest.mark.parametrize("M,N,K", [(16, 2112, 7168), (64, 7168, 2048), (4, 256, 512)])
def test_gemm_repeat_identical_and_workspace_left_zero(M, N, K):
    say(f"gemm repeat M={M} N={N} K={K}")
    g = np.random.default_rng(5)
    a = synth.f32_to_bf16_bits(g.standard_normal((M, K)).astype(np.float32))
    b = synth.f32_to_bf16_bits((g.standard_normal((N, K)) * 0.02).astype(np.float32))
    bq, bs = oracle.quant_mx(b)
    at, bp = to_dev_bf16(a), packed_b(bq, bs)
    outs = [bits_of(ops.gemm(at, bp, N)) for _ in range(6)]
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])
    wsz = ops.lib().gemm_a4w4_workspace_bytes(M, N, K)
    if wsz:
        # the split partial slots are zeroed again by every call
        used = ops.workspace(at.device, wsz)[:wsz].cpu().numpy()
        assert (used == 0).all()


# gemm_a4w4: the unfused comparator (A quantised by mxfp4_quant, then the GEMM on A_q).
# Where it runs the same kernel and tiling as the fused call (split-K for M <= 16;
# past 16 rows the skinny or the tiled kernel, when gemm_a4w4_fused_path names
# either) its C must be bit-identical; elsewhere within the oracle's tolerance. The
# skinny kernel's pre-quantised form with 4-, 8- and 16-row tiles, M and K tails.
A4W4_SHAPES = [(1, 16, 128), (4, 256, 512), (16, 2112, 7168), (3, 70, 352), (16, 130, 7232), (16, 130, 1088),
               (33, 64, 352), (64, 130, 2048), (65, 130, 288), (127, 257, 1056), (300, 33, 32), (256, 512, 4096),
               (17, 300, 1056), (40, 2000, 832), (100, 1000, 832), (257, 1024, 2048), (520, 4000, 704),
               (200, 4100, 1088)]


@pytest.mark.parametrize("M,N,K", A4W4_SHAPES)
def test_gemm_a4w4_matches_fused_and_oracle(M, N, K):
    say(f"gemm_a4w4 M={M} N={N} K={K}")
    g = np.random.default_rng(M * 5 + N * 3 + K)
    a = synth.f32_to_bf16_bits(g.standard_normal((M, K)).astype(np.float32))
    b = synth.f32_to_bf16_bits((g.standard_normal((N, K)) * 0.02).astype(np.float32))
    bq, bs = oracle.quant_mx(b)
    at, bp = to_dev_bf16(a), packed_b(bq, bs)
    aq, asc = ops.quant(at)
    c4 = bits_of(ops.gemm_a4w4(aq, asc, bp, N))
    cf = bits_of(ops.gemm(at, bp, N))
    path = ops.fused_path(M, N, K)
    if (path == "splitk") if M <= 16 else (path in ("skinny", "tiled")):
        assert np.array_equal(c4, cf)
    assert_in_tolerance(c4, oracle.gemm_ref(a, bq, bs), f"a4w4 M={M} N={N} K={K}")


# Mid-size M: the fused call takes the kernel its cost model estimates fastest
# (gemm_a4w4_fused_path). Each option against the oracle with M, N and K tails:
# the skinny kernel; the grouped kernel's skinny tiles of two, three and four
# 16-row sub-tiles (the last row tile partly or wholly past M); the tiled kernel.
MID_M = [((100, 1000, 832), "skinny"), ((257, 1024, 2048), "skinny"), ((200, 4100, 1088), "skinny_tiles"),
         ((180, 5000, 544), "skinny_tiles"), ((600, 2000, 3072), "skinny_tiles"), ((500, 4000, 1056), "skinny_tiles"),
         ((520, 4000, 704), "tiled")]


@pytest.mark.parametrize("shape,path", MID_M)
def test_fused_mid_m_kernels(shape, path):
    M, N, K = shape
    assert ops.fused_path(M, N, K) == path
    say(f"fused mid-M M={M} N={N} K={K} ({path})")
    g = np.random.default_rng(M + 7 * N + 3 * K)
    a = synth.f32_to_bf16_bits(g.standard_normal((M, K)).astype(np.float32))
    b = synth.f32_to_bf16_bits((g.standard_normal((N, K)) * 0.02).astype(np.float32))
    bq, bs = oracle.quant_mx(b)
    at, bp = to_dev_bf16(a), packed_b(bq, bs)
    c = bits_of(ops.gemm(at, bp, N))
    assert_in_tolerance(c, oracle.gemm_ref(a, bq, bs), f"M={M} N={N} K={K}")
    assert np.array_equal(bits_of(ops.gemm(at, bp, N)), c)  # repeat: the same bits


@pytest.mark.parametrize("M,N,K", [(16, 2112, 7168), (5, 100, 352), (130, 200, 416)])
def test_gemm_a4w4_strides_and_padding(M, N, K):
    """Row strides with padding that holds garbage (codes 0x77, scale bytes 0xFF = E8M0 NaN) must be
    ignored, including in a K tail; C's guard band stays untouched."""
    say(f"gemm_a4w4 strided M={M} N={N} K={K}")
    g = np.random.default_rng(13)
    a = synth.f32_to_bf16_bits(g.standard_normal((M, K)).astype(np.float32))
    b = synth.f32_to_bf16_bits((g.standard_normal((N, K)) * 0.02).astype(np.float32))
    bq, bs = oracle.quant_mx(b)
    rq, rs = oracle.quant_mx(a)
    ldaq, ldas, ldc = K // 2 + 48, K // 32 + 5, N + 8
    qbuf = np.full((M, ldaq), 0x77, np.uint8)
    qbuf[:, :K // 2] = rq
    sbuf = np.full((M, ldas), 0xFF, np.uint8)
    sbuf[:, :K // 32] = rs
    qd, sd = to_dev_u8(qbuf), to_dev_u8(sbuf)
    cbuf = torch.full((M + 2, ldc), 1234.0, dtype=torch.bfloat16, device="cuda")
    cview = cbuf[1:M + 1]
    bp = packed_b(bq, bs)
    wsz = ops.lib().gemm_a4w4_workspace_bytes(M, N, K)
    ws = ops.workspace(qd.device, wsz)
    rc = ops.lib().gemm_a4w4(qd.data_ptr(), ldaq, sd.data_ptr(), ldas, bp.data_ptr(), cview.data_ptr(), ldc, M, N, K,
                             ws.data_ptr() if wsz else None, ws.numel() if wsz else 0,
                             torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    cb = bits_of(cbuf)
    assert_in_tolerance(cb[1:M + 1, :N], oracle.gemm_ref(a, bq, bs), "a4w4 strided")
    guard = bits_of(torch.tensor([1234.0], dtype=torch.bfloat16))[0]
    assert (cb[0] == guard).all() and (cb[M + 1] == guard).all() and (cb[:, N:] == guard).all()


def test_grouped_ragged_small():
    say("grouped ragged small")
    g = np.random.default_rng(9)
    N, K = 100, 96
    Ms = [1, 70, 200, 129]
    a = [synth.f32_to_bf16_bits(g.standard_normal((m, K)).astype(np.float32)) for m in Ms]
    b = [synth.f32_to_bf16_bits((g.standard_normal((N, K)) * 0.02).astype(np.float32)) for _ in Ms]
    qs = [oracle.quant_mx(x) for x in b]
    cs = ops.grouped_gemm([to_dev_bf16(x) for x in a], [packed_b(*q) for q in qs], N)
    torch.cuda.synchronize()
    for x, (bq, bs), c in zip(a, qs, cs):
        assert_in_tolerance(bits_of(c), oracle.gemm_ref(x, bq, bs), f"M={x.shape[0]}")


def test_grouped_small_groups_mixed():
    """Groups of at most 64 rows take 16 x 128 tiles over the whole K (K split over the workgroup's waves),
    larger ones 128 x 512 tiles, in one launch: M tails (1, 17, 33, 63), the boundary (64 / 65), N not a
    multiple of 128 or 512, and a K tail on odd K/64. 26 large tiles (their id range padded to 32 with
    idle workgroups) ahead of 120 small ones."""
    say("grouped small groups mixed with large ones")
    g = np.random.default_rng(12)
    N, K = 1000, 832
    Ms = [1, 16, 17, 64, 65, 300, 33, 63, 1024, 100]
    a = [synth.f32_to_bf16_bits(g.standard_normal((m, K)).astype(np.float32)) for m in Ms]
    b = [synth.f32_to_bf16_bits((g.standard_normal((N, K)) * 0.02).astype(np.float32)) for _ in Ms]
    qs = [oracle.quant_mx(x) for x in b]
    cs = ops.grouped_gemm([to_dev_bf16(x) for x in a], [packed_b(*q) for q in qs], N)
    torch.cuda.synchronize()
    for x, (bq, bs), c in zip(a, qs, cs):
        assert_in_tolerance(bits_of(c), oracle.gemm_ref(x, bq, bs), f"M={x.shape[0]}")


# Small groups whose tiles of all rows would leave CUs idle while 16-row tiles would need a second round:
# the launch takes tiles of two (first case) or three (second) 16-row sub-tiles, so the last row tile of a
# 40-, 48- or 64-row group has sub-tiles wholly past its M (no loads, no stores). Odd K/64 tails.
@pytest.mark.parametrize("Ms,N,K", [([48, 40, 64, 17], 4096, 832), ([64, 48, 48, 48, 48], 4096, 352)])
def test_grouped_small_tiles_fewer_subtiles(Ms, N, K):
    say(f"grouped capped sub-tiles Ms={Ms} N={N} K={K}")
    g = np.random.default_rng(14)
    a = [synth.f32_to_bf16_bits(g.standard_normal((m, K)).astype(np.float32)) for m in Ms]
    b = [synth.f32_to_bf16_bits((g.standard_normal((N, K)) * 0.02).astype(np.float32)) for _ in Ms]
    qs = [oracle.quant_mx(x) for x in b]
    cs = ops.grouped_gemm([to_dev_bf16(x) for x in a], [packed_b(*q) for q in qs], N)
    torch.cuda.synchronize()
    for x, (bq, bs), c in zip(a, qs, cs):
        assert_in_tolerance(bits_of(c), oracle.gemm_ref(x, bq, bs), f"M={x.shape[0]}")


def tile_kinds(Ms, N, K):
    """Per group: "skinny" or "tiled", read from the dump layout (one copy per 128 or per 512 columns)."""
    arr = (ops.Group * len(Ms))()
    for i, m in enumerate(Ms):
        arr[i] = ops.Group(1 << 20, K, 1 << 20, 1 << 20, N, m)
    c = [ops.lib().grouped_gemm_a4w4_dump_copies(arr, len(Ms), N, K, i) for i in range(len(Ms))]
    return ["skinny" if ci == -(-N // 128) else "tiled" for ci in c]


# Groups of 65..512 rows on skinny tiles: the launch model moves them off 128 x 512 tiles when only a few
# such groups share the launch (several row tiles per column, M tails, odd K/64).
@pytest.mark.parametrize("Ms,N,K", [([128, 128], 4096, 7168), ([100, 200, 300], 2000, 1056), ([70, 16, 250], 3000, 544)])
def test_grouped_mid_groups_on_skinny_tiles(Ms, N, K):
    assert tile_kinds(Ms, N, K) == ["skinny"] * len(Ms)
    say(f"grouped mid groups Ms={Ms} N={N} K={K}")
    g = np.random.default_rng(15)
    a = [synth.f32_to_bf16_bits(g.standard_normal((m, K)).astype(np.float32)) for m in Ms]
    b = [synth.f32_to_bf16_bits((g.standard_normal((N, K)) * 0.02).astype(np.float32)) for _ in Ms]
    qs = [oracle.quant_mx(x) for x in b]
    cs = ops.grouped_gemm([to_dev_bf16(x) for x in a], [packed_b(*q) for q in qs], N)
    torch.cuda.synchronize()
    for x, (bq, bs), c in zip(a, qs, cs):
        assert_in_tolerance(bits_of(c), oracle.gemm_ref(x, bq, bs), f"M={x.shape[0]}")


# Small groups only, whose 16-row tiles all fit one round of workgroups: the launch runs the 16-wave skinny
# tiles, 128 columns wide, or 64 when 128-column tiles would fill at most half a round (M tails 1, 17, 33,
# 5; ragged N; a K tail on odd K/64).
@pytest.mark.parametrize("Ms", [[1, 16, 17, 33, 64, 5], [1, 17, 33, 5]])
def test_grouped_small_only_one_round(Ms):
    say(f"grouped small only, one round, Ms={Ms}")
    g = np.random.default_rng(16)
    N, K = 2000, 1056
    assert sum(-(-m // 16) for m in Ms) * -(-N // 128) <= 256
    a = [synth.f32_to_bf16_bits(g.standard_normal((m, K)).astype(np.float32)) for m in Ms]
    b = [synth.f32_to_bf16_bits((g.standard_normal((N, K)) * 0.02).astype(np.float32)) for _ in Ms]
    qs = [oracle.quant_mx(x) for x in b]
    cs = ops.grouped_gemm([to_dev_bf16(x) for x in a], [packed_b(*q) for q in qs], N)
    torch.cuda.synchronize()
    for x, (bq, bs), c in zip(a, qs, cs):
        assert_in_tolerance(bits_of(c), oracle.gemm_ref(x, bq, bs), f"M={x.shape[0]}")


def test_grouped_small_subtiles_ragged():
    """Small groups whose 16-row tiles would not fit one round of workgroups take one tile of all their
    rows (one to four 16-row sub-tiles sharing each B load): M 5, 17, 33, 48, 57, 64, N with a tail of 8 columns
    past the last 128, K with a tail on odd K/64."""
    say("grouped small groups, multi-row tiles")
    g = np.random.default_rng(13)
    N, K = 8200, 832
    Ms = [17, 33, 48, 5, 57, 64]
    a = [synth.f32_to_bf16_bits(g.standard_normal((m, K)).astype(np.float32)) for m in Ms]
    b = [synth.f32_to_bf16_bits((g.standard_normal((N, K)) * 0.02).astype(np.float32)) for _ in Ms]
    qs = [oracle.quant_mx(x) for x in b]
    cs = ops.grouped_gemm([to_dev_bf16(x) for x in a], [packed_b(*q) for q in qs], N)
    torch.cuda.synchronize()
    for x, (bq, bs), c in zip(a, qs, cs):
        assert_in_tolerance(bits_of(c), oracle.gemm_ref(x, bq, bs), f"M={x.shape[0]}")


def _tile_rows(m):
    """First and last row of every 128-row tile of an M-row group (whole rows: every column tile)."""
    return np.unique(np.concatenate([np.arange(0, m, 128), np.minimum(np.arange(127, m + 127, 128), m - 1)]))


# More 128 x 512 tiles than the 256 CUs (a second round of workgroups): 264 tiles over 9 K steps (odd K/64,
# a K tail); 320 tiles over 3 K steps; 306 tiles over one K step with a ragged N.
@pytest.mark.parametrize("Ms,N,K", [([640, 512, 384, 1024, 256, 200, 700, 300], 4096, 1056),
                                    ([1024, 1024, 1024, 1024, 1000], 4096, 352),
                                    ([1200, 1200, 1200, 1200, 1200, 100], 3000, 32)])
def test_grouped_more_tiles_than_cus(Ms, N, K):
    say(f"grouped Ms {Ms} N{N} K{K}")
    g = np.random.default_rng(41)
    a = [synth.f32_to_bf16_bits(g.standard_normal((m, K)).astype(np.float32)) for m in Ms]
    b = [synth.f32_to_bf16_bits((g.standard_normal((N, K)) * 0.02).astype(np.float32)) for _ in Ms]
    qs = [oracle.quant_mx(x) for x in b]
    cs = ops.grouped_gemm([to_dev_bf16(x) for x in a], [packed_b(*q) for q in qs], N)
    torch.cuda.synchronize()
    for gi, (x, (bq, bs), c) in enumerate(zip(a, qs, cs)):
        rows = _tile_rows(x.shape[0])
        assert_in_tolerance(bits_of(c)[rows], oracle.gemm_ref(x[rows], bq, bs), f"group {gi} (M={x.shape[0]})")


def test_grouped_on_a_side_stream():
    """The grouped call reads the device's CU count through the stream it is given (a non-default stream
    here); small and large groups, the same C as on the default stream."""
    say("grouped on a side stream")
    g = np.random.default_rng(14)
    N, K = 600, 512
    Ms = [9, 40, 130, 700]
    a = [to_dev_bf16(synth.f32_to_bf16_bits(g.standard_normal((m, K)).astype(np.float32))) for m in Ms]
    b = [oracle.quant_mx(synth.f32_to_bf16_bits((g.standard_normal((N, K)) * 0.02).astype(np.float32)))
         for _ in Ms]
    bp = [packed_b(*q) for q in b]
    ref = [bits_of(c) for c in ops.grouped_gemm(a, bp, N)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        cs = ops.grouped_gemm(a, bp, N)
    side.synchronize()
    for r, c in zip(ref, cs):
        assert np.array_equal(r, bits_of(c))


@pytest.mark.timeout(600)
def test_grouped_decode_workload():
    """The decode-sized grouped workload (8 groups of 8..64 rows, N4096 K7168), every row."""
    say("grouped_decode workload")
    w = synth.workload("grouped_decode", synth.default_seed("grouped_decode"))
    qs = quant_groups_in_pool(w["B"])
    cs = ops.grouped_gemm([to_dev_bf16(a) for a in w["A"]], [packed_b(bq, bs) for bq, bs in qs], w["N"])
    torch.cuda.synchronize()
    for g, (a, (bq, bs), c) in enumerate(zip(w["A"], qs, cs)):
        assert_in_tolerance(bits_of(c), oracle.gemm_ref(a, bq, bs), f"group {g} (M={a.shape[0]})")


def test_gemm_two_streams_use_their_own_workspaces():
    """Split-K calls (M <= 16, partials through the workspace) issued on two streams at once: each stream
    has its own workspace, both results equal the one-stream results bit for bit, and both workspaces
    are left zeroed."""
    say("gemm on two streams")
    M, N, K = 16, 2112, 7168
    g = np.random.default_rng(41)
    a1 = synth.f32_to_bf16_bits(g.standard_normal((M, K)).astype(np.float32))
    a2 = synth.f32_to_bf16_bits(g.standard_normal((M, K)).astype(np.float32))
    b = synth.f32_to_bf16_bits((g.standard_normal((N, K)) * 0.02).astype(np.float32))
    bq, bs = oracle.quant_mx(b)
    bp = packed_b(bq, bs)
    t1, t2 = to_dev_bf16(a1), to_dev_bf16(a2)
    r1, r2 = bits_of(ops.gemm(t1, bp, N)), bits_of(ops.gemm(t2, bp, N))
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    outs1, outs2 = [], []
    for _ in range(20):
        with torch.cuda.stream(s1):
            outs1.append(ops.gemm(t1, bp, N))
        with torch.cuda.stream(s2):
            outs2.append(ops.gemm(t2, bp, N))
    torch.cuda.synchronize()
    for c in outs1:
        assert np.array_equal(bits_of(c), r1)
    for c in outs2:
        assert np.array_equal(bits_of(c), r2)
    wsz = ops.lib().gemm_a4w4_workspace_bytes(M, N, K)
    w1 = ops.workspace(t1.device, wsz, s1.cuda_stream)
    w2 = ops.workspace(t2.device, wsz, s2.cuda_stream)
    assert w1.data_ptr() != w2.data_ptr()
    assert (w1[:wsz].cpu().numpy() == 0).all() and (w2[:wsz].cpu().numpy() == 0).all()
    assert_in_tolerance(r1, oracle.gemm_ref(a1, bq, bs), "stream 1")
