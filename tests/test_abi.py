"""The C ABI without a GPU: every declared symbol is exported, size queries
follow the documented layout, and every validation error is returned before any
HIP call (nothing is launched, so no device is needed)."""
import ctypes
import os
import re

import pytest

from mxfp4_block_scaled_02_amd import ops

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "mxfp4.h")


def cdiv(a, b):
    return (a + b - 1) // b


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?(?:int64_t|int|size_t|char\s*\*|const char\s*\*)\s*\*?\s*(\w+)\s*\(",
                                 text, flags=re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    assert set(names) == set(ops.EXPORTED)


def test_library_exports_every_declared_symbol():
    L = ops.lib()
    for name in declared_functions():
        assert hasattr(L, name), name


def test_status_strings():
    L = ops.lib()
    for code, name in ops.STATUS.items():
        assert L.mxfp4_status_str(code).decode().startswith(name)
    assert L.mxfp4_status_str(99) == b"unknown mxfp4 status"


@pytest.mark.parametrize("N,K", [(1, 32), (16, 128), (17, 160), (2112, 7168), (4096, 7168), (7168, 2048)])
def test_pack_B_bytes_formula(N, K):
    NT, KU = cdiv(N, 32), cdiv(K, 64)
    KG = cdiv(KU, 4)
    assert ops.lib().mxfp4_pack_B_bytes(N, K) == NT * KU * 1024 + NT * KG * 256


@pytest.mark.parametrize("N,K", [(0, 32), (16, 0), (16, 48), (-1, 64)])
def test_pack_B_bytes_invalid_is_zero(N, K):
    assert ops.lib().mxfp4_pack_B_bytes(N, K) == 0


def _splitk_range(M, N, K):
    """Split-K workspace (M <= 16), from the header's geometry: T = ceil(ceil(N/16)/4)
    tiles of 64 columns and S splits with ceil(KT/8) <= S <= min(KT, 64), KT =
    ceil(K/128); the fp32 partials (16 x 64 per tile) of S-1 splits, i.e.
    T*(S-1)*4096 bytes. Returns (T, smin, smax), or None when split-K is not used."""
    KT = -(-K // 128)
    T = -(-(-(-N // 16)) // 4)
    smin = -(-KT // 8)
    if smin > 64:
        return None
    return T, smin, min(KT, 64)


def test_workspace_sizes_are_consistent():
    L = ops.lib()
    assert L.gemm_a4w4_workspace_bytes(0, 16, 32) == 0
    assert L.gemm_a4w4_workspace_bytes(4, 16, 48) == 0  # invalid K
    for M, N, K in [(4, 256, 512), (16, 2112, 7168), (1, 4096, 7168), (16, 64, 65536), (1, 1, 32), (16, 130, 7232)]:
        T, smin, smax = _splitk_range(M, N, K)
        w = L.gemm_a4w4_workspace_bytes(M, N, K)
        assert w % (T * 4096) == 0 and smin <= w // (T * 4096) + 1 <= smax, (M, N, K, w)
    assert L.gemm_a4w4_workspace_bytes(16, 2112, 7168) > 0  # K = 7168 needs at least 7 splits
    assert L.gemm_a4w4_workspace_bytes(16, 64, 65536) == 63 * 4096  # 512 K steps: 64 splits
    assert L.gemm_a4w4_workspace_bytes(16, 48, 66560) == 0  # more than 64 splits: no split-K
    for M, N, K in [(17, 2112, 7168), (64, 7168, 2048), (4096, 4096, 7168)]:
        assert L.gemm_a4w4_workspace_bytes(M, N, K) == 0


P = 1 << 20  # a fake, 256-byte aligned "device pointer": validation never dereferences it
OK_Q = dict(x=P, ldx=64, q=P, ldq=32, s=P, lds=2, M=4, K=64)


@pytest.mark.parametrize("change,status", [
    (dict(x=None), 1), (dict(q=None), 1), (dict(s=None), 1),
    (dict(M=0), 2), (dict(K=0), 2), (dict(K=48), 2), (dict(ldx=32), 2), (dict(ldq=16), 2), (dict(lds=1), 2),
    (dict(x=P + 2), 3), (dict(q=P + 8), 3), (dict(ldx=68), 3), (dict(ldq=40), 3),
    (dict(M=1 << 30, K=1 << 30, ldx=1 << 30, ldq=1 << 29, lds=1 << 25), 2),  # grid past 2^31 workgroups
])
def test_quant_validation(change, status):
    a = dict(OK_Q, **change)
    got = ops.lib().mxfp4_quant(a["x"], a["ldx"], a["q"], a["ldq"], a["s"], a["lds"], a["M"], a["K"], None)
    assert got == status


OK_R = dict(x=P, ldx=64, w=P, eps=1e-6, q=P, ldq=32, s=P, lds=2, M=4, K=64)


@pytest.mark.parametrize("change,status", [
    (dict(x=None), 1), (dict(w=None), 1), (dict(q=None), 1), (dict(s=None), 1),
    (dict(M=0), 2), (dict(K=0), 2), (dict(K=48), 2), (dict(ldx=32), 2), (dict(ldq=16), 2), (dict(lds=1), 2),
    (dict(eps=0.0), 8), (dict(eps=-1e-6), 8), (dict(eps=float("nan")), 8), (dict(eps=float("inf")), 8),
    (dict(x=P + 2), 3), (dict(w=P + 8), 3), (dict(q=P + 2), 3), (dict(ldx=68), 3), (dict(ldq=34), 3),
])
def test_rmsnorm_quant_validation(change, status):
    a = dict(OK_R, **change)
    got = ops.lib().mxfp4_rmsnorm_quant(a["x"], a["ldx"], a["w"], a["eps"], a["q"], a["ldq"], a["s"], a["lds"],
                                        a["M"], a["K"], None)
    assert got == status


@pytest.mark.parametrize("change,status", [
    (dict(bq=None), 1), (dict(out=None), 1), (dict(N=0), 2), (dict(K=40), 2),
    (dict(bq=P + 4), 3), (dict(out=P + 1), 3), (dict(out_bytes=1000), 7),
    (dict(N=1 << 30, K=1 << 30, out_bytes=1 << 62), 2),  # grid past 2^31 workgroups
])
def test_pack_B_validation(change, status):
    a = dict(dict(bq=P, bs=P, N=16, K=128, out=P, out_bytes=2 * 1024 + 256), **change)
    got = ops.lib().mxfp4_pack_B(a["bq"], a["bs"], a["N"], a["K"], a["out"], a["out_bytes"], None)
    assert got == status


OK_G = dict(A=P, lda=7168, Bp=P, C=P, ldc=2112, M=16, N=2112, K=7168, ws=P, wsb=1 << 30)


@pytest.mark.parametrize("change,status", [
    (dict(A=None), 1), (dict(Bp=None), 1), (dict(C=None), 1),
    (dict(M=0), 2), (dict(N=0), 2), (dict(K=7000), 2), (dict(lda=7000), 2), (dict(ldc=2000), 2),
    (dict(M=1 << 31), 2),
    # 32-bit buffer offsets: a 128-row A window and a packed 32-column B tile stay below 2^31 bytes
    (dict(lda=1 << 23), 2), (dict(lda=8388552), 2), (dict(M=17, lda=1 << 23), 2),
    (dict(M=4096, lda=1 << 23), 2), (dict(K=1 << 27, lda=1 << 27), 2), (dict(K=(1 << 27) - 64, lda=(1 << 27) - 64), 2),
    (dict(A=P + 2), 3), (dict(lda=7172), 3), (dict(Bp=P + 8), 3), (dict(C=P + 1), 3),
    (dict(ws=None), 4), (dict(wsb=1024), 4), (dict(ws=P + 16), 3),
])
def test_gemm_validation(change, status):
    a = dict(OK_G, **change)
    got = ops.lib().gemm_a4w4_fused(a["A"], a["lda"], a["Bp"], a["C"], a["ldc"], a["M"], a["N"], a["K"], a["ws"],
                                    a["wsb"], None)
    assert got == status


@pytest.mark.parametrize("change,status", [
    (dict(A=None), 1), (dict(Bp=None), 1), (dict(C=None), 1),
    (dict(M=0), 2), (dict(K=7000), 2), (dict(lda=7000), 2), (dict(lda=1 << 23), 2),
    (dict(A=P + 2), 3), (dict(C=P + 1), 3),
    # split-K needs 17 tiles x 63 splits x 4 KB of partials, more than the fixed scratch holds
    (dict(M=16, N=1088, K=65536, lda=65536, ldc=1088), 4),
])
def test_gemm_noalloc_validation(change, status):
    a = dict(OK_G, **change)
    got = ops.lib().gemm_a4w4_fused_noalloc(a["A"], a["lda"], a["Bp"], a["C"], a["ldc"], a["M"], a["N"], a["K"], None)
    assert got == status


def test_noalloc_scratch_limit_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define MXFP4_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    limit = int(m.group(1)) << int(m.group(2))
    L = ops.lib()
    assert L.gemm_a4w4_workspace_bytes(16, 1088, 65536) > limit
    assert 0 < L.gemm_a4w4_workspace_bytes(16, 2112, 7168) <= limit


OK_Q4 = dict(Aq=P, ldaq=3584, As=P, ldas=224, Bp=P, C=P, ldc=2112, M=16, N=2112, K=7168, ws=P, wsb=1 << 30)


@pytest.mark.parametrize("change,status", [
    (dict(Aq=None), 1), (dict(As=None), 1), (dict(Bp=None), 1), (dict(C=None), 1),
    (dict(M=0), 2), (dict(K=7000), 2), (dict(ldaq=3000), 2), (dict(ldas=200), 2), (dict(ldc=2000), 2),
    (dict(ldaq=1 << 25), 2),
    (dict(K=1 << 27, ldaq=1 << 24, ldas=1 << 22), 2),  # a packed B tile of ceil(K/64) KB reaches 2^31 bytes
    (dict(Aq=P + 8), 3), (dict(ldaq=3592), 3), (dict(Bp=P + 8), 3), (dict(C=P + 1), 3),
    (dict(ws=None), 4), (dict(wsb=1024), 4), (dict(ws=P + 16), 3),
])
def test_gemm_a4w4_validation(change, status):
    a = dict(OK_Q4, **change)
    got = ops.lib().gemm_a4w4(a["Aq"], a["ldaq"], a["As"], a["ldas"], a["Bp"], a["C"], a["ldc"], a["M"], a["N"],
                              a["K"], a["ws"], a["wsb"], None)
    assert got == status


def test_grouped_validation():
    L = ops.lib()
    g = (ops.Group * 2)()
    g[0] = ops.Group(P, 7168, P, P, 4096, 128)
    g[1] = ops.Group(P, 7168, P, P, 4096, 0)  # bad M in group 1
    assert L.grouped_gemm_a4w4(g, 2, 4096, 7168, None, 0, None) == 2
    assert L.grouped_gemm_a4w4(g, 0, 4096, 7168, None, 0, None) == 5
    assert L.grouped_gemm_a4w4(g, 33, 4096, 7168, None, 0, None) == 5
    assert L.grouped_gemm_a4w4(None, 1, 4096, 7168, None, 0, None) == 1
    g[1] = ops.Group(P, 7168, None, P, 4096, 64)
    assert L.grouped_gemm_a4w4(g, 2, 4096, 7168, None, 0, None) == 1
    g[1] = ops.Group(P + 2, 7168, P, P, 4096, 64)
    assert L.grouped_gemm_a4w4(g, 2, 4096, 7168, None, 0, None) == 3
    g[1] = ops.Group(P, 1 << 23, P, P, 4096, 64)  # a 128-row window of A past 2^31 bytes
    assert L.grouped_gemm_a4w4(g, 2, 4096, 7168, None, 0, None) == 2


def test_small_m_kernel_choice():
    """For M <= 16 the fused call runs the split-K kernel (dump copies = its 64-column tiles) unless the split
    needs a hand-off and the skinny kernel (16-column tiles, K split over one workgroup's waves) is estimated
    faster: wide N. The verification dump's size shows which one a shape takes."""
    L = ops.lib()
    row = lambda K: K // 2 + K // 32
    splitk = [(16, 2112, 7168), (16, 264, 7168), (4, 256, 512), (1, 16, 128), (16, 130, 7232), (16, 1088, 65536),
              (16, 4096, 7168)]
    for M, N, K in splitk:
        assert L.gemm_a4w4_fused_dump_bytes(M, N, K) == cdiv(cdiv(N, 16), 4) * M * row(K), (M, N, K)
    skinny = [(1, 4096, 7168, 1), (8, 4096, 7168, 2), (16, 7168, 2048, 4), (2, 4096, 4096, 1)]  # (.., NB)
    for M, N, K, nb in skinny:
        assert L.gemm_a4w4_fused_dump_bytes(M, N, K) == cdiv(cdiv(N, 16), nb) * M * row(K), (M, N, K)
    # gemm_a4w4 always runs split-K at M <= 16: its workspace size is that kernel's
    assert L.gemm_a4w4_workspace_bytes(1, 4096, 7168) > 0


def test_fused_kernel_choice_mid_m():
    """Past 64 rows the fused call keeps the tiled kernel unless its cost model estimates the skinny kernel or
    the grouped kernel's skinny tiles at least 15 % faster: a few hundred rows leave most 128 x 512 tiles'
    CUs idle. The choice depends on (M, N, K) alone, and the verification dump's size follows it (one copy
    per 128 columns for the skinny tiles, per 512 for the tiled kernel)."""
    L = ops.lib()
    row = lambda K: K // 2 + K // 32
    want = {(16, 2112, 7168): "splitk", (1, 4096, 7168): "skinny", (64, 7168, 2048): "skinny",
            (65, 4096, 7168): "skinny", (128, 4096, 7168): "skinny", (128, 1024, 4096): "skinny",
            (192, 4096, 7168): "skinny_tiles", (512, 4096, 7168): "skinny_tiles", (256, 7168, 2048): "skinny_tiles",
            (512, 2112, 7168): "skinny_tiles",
            (768, 4096, 7168): "tiled", (4096, 4096, 7168): "tiled", (512, 7168, 2048): "tiled",
            (5000, 4096, 7168): "tiled"}
    for (M, N, K), path in want.items():
        assert ops.fused_path(M, N, K) == path, (M, N, K)
        if M > 64 and path != "skinny":
            per = 128 if path == "skinny_tiles" else 512
            assert L.gemm_a4w4_fused_dump_bytes(M, N, K) == cdiv(N, per) * M * row(K), (M, N, K)
    for M, N, K in [(0, 16, 32), (16, 0, 32), (16, 16, 48), (16, 16, 0)]:
        assert L.gemm_a4w4_fused_path(M, N, K) == 0
        with pytest.raises(ValueError):
            ops.fused_path(M, N, K)


def test_grouped_dump_layout():
    """A group on skinny tiles has one dump copy per 128 columns (per 64 when only small groups share the
    launch and their 128-column tiles would fill at most half a round), one on 128 x 512 tiles one per 512.
    Groups of at most 64 rows always take skinny tiles; a group of up to 512 rows takes them too when the
    launch model estimates the whole launch faster so (here: one or two mid-size groups alone), which makes
    its copy count a function of the whole list."""
    L = ops.lib()

    def copies(Ms, N, K):
        g = (ops.Group * len(Ms))()
        for i, M in enumerate(Ms):
            g[i] = ops.Group(P, K, P, P, N, M)
        c = [L.grouped_gemm_a4w4_dump_copies(g, len(Ms), N, K, i) for i in range(len(Ms))]
        assert L.grouped_gemm_a4w4_dump_bytes(g, len(Ms), N, K) == sum(ci * M * (K // 2 + K // 32)
                                                                        for ci, M in zip(c, Ms))
        return c

    assert copies([1, 16, 48, 64], 4096, 7168) == [32] * 4
    assert copies([16, 100], 1000, 832) == [16, 16]   # the 100-row group too: skinny tiles, 64 columns (half a round)
    assert copies([128, 128], 4096, 7168) == [32, 32]                   # 16 tiled tiles for 256 CUs: skinny
    assert copies([448, 384, 704, 384, 1024, 128, 256, 640], 4096, 7168) == [8] * 8   # 256 tiled tiles: kept
    assert copies([1024, 128], 4096, 7168) == [8, 8]                    # the 1024-row group bounds it: kept
    assert copies([600, 64], 4096, 7168) == [8, 32]                     # past 512 rows: always tiled
    assert copies([16, 200, 64], 1000, 832) == [8, 8, 8]                # 144 tiles of 128 columns: kept
    assert copies([1, 17, 33, 5], 2000, 1056) == [32] * 4                 # 112 tiles of 128 columns: 64 instead
    g = (ops.Group * 2)()
    g[0], g[1] = ops.Group(P, 64, P, P, 64, 16), ops.Group(P, 64, P, P, 64, 0)
    assert L.grouped_gemm_a4w4_dump_copies(g, 2, 64, 64, 0) == 0         # an invalid list
    g[1] = ops.Group(P, 64, P, P, 64, 16)
    assert L.grouped_gemm_a4w4_dump_copies(g, 2, 64, 64, 2) == 0         # g out of range
    assert L.grouped_gemm_a4w4_dump_copies(g, 2, 0, 64, 0) == 0 and L.grouped_gemm_a4w4_dump_copies(g, 2, 64, 48, 0) == 0


def _mnk(**kw):
    d = dict(A=P, lda=512, strideA=0, Bp=P, strideB=0, C=P, ldc=64, strideC=0, M=16, N=64, K=512, L=1)
    d.update(kw)
    return ops.GroupMnk(d["A"], d["lda"], d["strideA"], d["Bp"], d["strideB"], d["C"], d["ldc"], d["strideC"],
                        d["M"], d["N"], d["K"], d["L"])


@pytest.mark.parametrize("groups,status", [
    ([_mnk(A=None)], 1), ([_mnk(C=None)], 1),
    ([_mnk(L=0)], 2), ([_mnk(K=48)], 2), ([_mnk(lda=256)], 2), ([_mnk(ldc=32)], 2), ([_mnk(M=0)], 2),
    ([_mnk(A=P + 8)], 3), ([_mnk(Bp=P + 4)], 3), ([_mnk(lda=516)], 3),
    ([_mnk(lda=1 << 23)], 2),  # 32-bit buffer offsets over a 128-row A window
    # batches: C slices must not overlap, B slices must hold a packed image, strides keep alignment
    ([_mnk(L=2, strideA=512 * 16, strideB=1 << 20, strideC=16 * 64 - 1)], 2),
    ([_mnk(L=2, strideA=512 * 16, strideB=100, strideC=16 * 64)], 2),
    ([_mnk(L=2, strideA=-8, strideB=1 << 20, strideC=16 * 64)], 2),
    ([_mnk(L=2, strideA=4, strideB=1 << 20, strideC=16 * 64)], 3),
    ([_mnk(L=2, strideA=512 * 16, strideB=(1 << 20) + 4, strideC=16 * 64)], 3),
    # at most 32 problems in all
    ([_mnk(L=20, strideA=8192, strideB=1 << 20, strideC=1024), _mnk(L=13, strideA=8192, strideB=1 << 20,
                                                                      strideC=1024)], 5),
])
def test_grouped_mnk_validation(groups, status):
    arr = (ops.GroupMnk * len(groups))(*groups)
    assert ops.lib().grouped_gemm_a4w4_mnk(arr, len(groups), None) == status


def test_grouped_mnk_rejects_empty_list():
    assert ops.lib().grouped_gemm_a4w4_mnk(None, 1, None) == 1
    arr = (ops.GroupMnk * 1)(_mnk())
    assert ops.lib().grouped_gemm_a4w4_mnk(arr, 0, None) == 5


def _nv(**kw):
    d = dict(Aq=P, lda=256, strideA=0, As=P, ldas=32, strideAs=0, Bq=P, ldb=256, strideB=0, Bs=P, ldbs=32,
             strideBs=0, C=P, ldc=64, strideC=0, M=16, N=64, K=512, L=1)
    d.update(kw)
    return ops.GroupNv(*(d[f] for f, _ in ops.GroupNv._fields_))


@pytest.mark.parametrize("groups,status", [
    ([_nv(Aq=None)], 1), ([_nv(As=None)], 1), ([_nv(Bs=None)], 1), ([_nv(C=None)], 1),
    ([_nv(L=0)], 2), ([_nv(K=40)], 2), ([_nv(K=0)], 2), ([_nv(M=0)], 2), ([_nv(N=0)], 2),
    ([_nv(lda=240)], 2), ([_nv(ldas=30)], 2), ([_nv(ldb=128)], 2), ([_nv(ldbs=16)], 2), ([_nv(ldc=63)], 2),
    ([_nv(M=1 << 24, lda=1 << 8)], 2),  # (M + 128) * lda reaches 2^31
    ([_nv(Aq=P + 4)], 3), ([_nv(Bq=P + 12)], 3), ([_nv(lda=260)], 3), ([_nv(ldb=258)], 3), ([_nv(C=P + 1)], 3),
    # batches: C slices must not overlap; strides keep alignment
    ([_nv(L=2, strideA=4096, strideAs=512, strideB=16384, strideBs=2048, strideC=16 * 64 - 1)], 2),
    ([_nv(L=2, strideA=-16, strideAs=512, strideB=16384, strideBs=2048, strideC=16 * 64)], 2),
    ([_nv(L=2, strideA=4100, strideAs=512, strideB=16384, strideBs=2048, strideC=16 * 64)], 3),
    ([_nv(L=2, strideA=4096, strideAs=512, strideB=16386, strideBs=2048, strideC=16 * 64)], 3),
    # at most 32 problems in all
    ([_nv(L=20, strideA=4096, strideAs=512, strideB=16384, strideBs=2048, strideC=1024),
      _nv(L=13, strideA=4096, strideAs=512, strideB=16384, strideBs=2048, strideC=1024)], 5),
])
def test_grouped_nvfp4_validation(groups, status):
    arr = (ops.GroupNv * len(groups))(*groups)
    assert ops.lib().grouped_gemm_nvfp4(arr, len(groups), None) == status


def test_grouped_nvfp4_rejects_empty_list():
    assert ops.lib().grouped_gemm_nvfp4(None, 1, None) == 1
    arr = (ops.GroupNv * 1)(_nv())
    assert ops.lib().grouped_gemm_nvfp4(arr, 0, None) == 5
