"""Thin ctypes binding of libmxfp4.so (C ABI in include/mxfp4.h).

Argument marshalling only: torch supplies device memory and the current
stream; every step of the computation runs in the library's HIP kernels. There
is no fallback: if the library is missing or a call returns a non-zero status,
these functions raise.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

# MXFP4_LIB names another build of the same library (the sanitizer check build);
# it must exist like the default one.
_LIB_PATH = os.environ.get("MXFP4_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmxfp4.so")
_lib = None
_lock = threading.Lock()

MXFP4_MAX_GROUPS = 32
STATUS = {0: "MXFP4_OK", 1: "MXFP4_ERR_NULL", 2: "MXFP4_ERR_SHAPE", 3: "MXFP4_ERR_ALIGN", 4: "MXFP4_ERR_WORKSPACE",
          5: "MXFP4_ERR_TOO_MANY_GROUPS", 6: "MXFP4_ERR_HIP", 7: "MXFP4_ERR_BUFFER", 8: "MXFP4_ERR_ARG"}
EXPORTED = ["mxfp4_status_str", "mxfp4_quant", "mxfp4_rmsnorm_quant", "mxfp4_pack_B_bytes", "mxfp4_pack_B",
            "gemm_a4w4_workspace_bytes", "gemm_a4w4_fused", "gemm_a4w4_fused_path", "gemm_a4w4_fused_noalloc",
            "gemm_a4w4_fused_dump_bytes",
            "gemm_a4w4_fused_dump",
            "gemm_a4w4", "grouped_gemm_a4w4_workspace_bytes", "grouped_gemm_a4w4", "grouped_gemm_a4w4_dump_bytes",
            "grouped_gemm_a4w4_dump_copies", "grouped_gemm_a4w4_dump", "grouped_gemm_a4w4_mnk", "grouped_gemm_nvfp4"]


class Mxfp4Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {lib().mxfp4_status_str(status).decode()} (status {status})")


class GroupMnk(ctypes.Structure):
    """mirror of mxfp4_group_mnk"""
    _fields_ = [("A", ctypes.c_void_p), ("lda", ctypes.c_int64), ("strideA", ctypes.c_int64),
                ("Bp", ctypes.c_void_p), ("strideB", ctypes.c_int64), ("C", ctypes.c_void_p), ("ldc", ctypes.c_int64),
                ("strideC", ctypes.c_int64), ("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
                ("L", ctypes.c_int64)]


class GroupNv(ctypes.Structure):
    """mirror of nvfp4_group"""
    _fields_ = [("Aq", ctypes.c_void_p), ("lda", ctypes.c_int64), ("strideA", ctypes.c_int64),
                ("As", ctypes.c_void_p), ("ldas", ctypes.c_int64), ("strideAs", ctypes.c_int64),
                ("Bq", ctypes.c_void_p), ("ldb", ctypes.c_int64), ("strideB", ctypes.c_int64),
                ("Bs", ctypes.c_void_p), ("ldbs", ctypes.c_int64), ("strideBs", ctypes.c_int64),
                ("C", ctypes.c_void_p), ("ldc", ctypes.c_int64), ("strideC", ctypes.c_int64),
                ("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64), ("L", ctypes.c_int64)]


class Group(ctypes.Structure):
    """mirror of mxfp4_group"""
    _fields_ = [("A", ctypes.c_void_p), ("lda", ctypes.c_int64), ("Bp", ctypes.c_void_p), ("C", ctypes.c_void_p),
                ("ldc", ctypes.c_int64), ("M", ctypes.c_int64)]


def lib() -> ctypes.CDLL:
    """Load libmxfp4.so (once) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is not built; run `python -m mxfp4_block_scaled_02_amd.build`")
        L = ctypes.CDLL(_LIB_PATH)
        vp, i64, sz, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int
        L.mxfp4_status_str.argtypes, L.mxfp4_status_str.restype = [i32], ctypes.c_char_p
        L.mxfp4_quant.argtypes, L.mxfp4_quant.restype = [vp, i64, vp, i64, vp, i64, i64, i64, vp], i32
        L.mxfp4_rmsnorm_quant.argtypes = [vp, i64, vp, ctypes.c_float, vp, i64, vp, i64, i64, i64, vp]
        L.mxfp4_rmsnorm_quant.restype = i32
        L.mxfp4_pack_B_bytes.argtypes, L.mxfp4_pack_B_bytes.restype = [i64, i64], sz
        L.mxfp4_pack_B.argtypes, L.mxfp4_pack_B.restype = [vp, vp, i64, i64, vp, sz, vp], i32
        L.gemm_a4w4_workspace_bytes.argtypes, L.gemm_a4w4_workspace_bytes.restype = [i64, i64, i64], sz
        L.gemm_a4w4_fused.argtypes = [vp, i64, vp, vp, i64, i64, i64, i64, vp, sz, vp]
        L.gemm_a4w4_fused.restype = i32
        L.gemm_a4w4_fused_path.argtypes, L.gemm_a4w4_fused_path.restype = [i64, i64, i64], i32
        L.gemm_a4w4_fused_noalloc.argtypes = [vp, i64, vp, vp, i64, i64, i64, i64, vp]
        L.gemm_a4w4_fused_noalloc.restype = i32
        L.gemm_a4w4_fused_dump_bytes.argtypes, L.gemm_a4w4_fused_dump_bytes.restype = [i64, i64, i64], sz
        L.gemm_a4w4_fused_dump.argtypes = [vp, i64, vp, vp, i64, i64, i64, i64, vp, sz, vp, sz, vp]
        L.gemm_a4w4_fused_dump.restype = i32
        L.grouped_gemm_a4w4_dump_bytes.argtypes = [ctypes.POINTER(Group), i32, i64, i64]
        L.grouped_gemm_a4w4_dump_bytes.restype = sz
        L.grouped_gemm_a4w4_dump_copies.argtypes = [ctypes.POINTER(Group), i32, i64, i64, i32]
        L.grouped_gemm_a4w4_dump_copies.restype = i64
        L.grouped_gemm_a4w4_dump.argtypes = [ctypes.POINTER(Group), i32, i64, i64, vp, sz, vp, sz, vp]
        L.grouped_gemm_a4w4_dump.restype = i32
        L.gemm_a4w4.argtypes = [vp, i64, vp, i64, vp, vp, i64, i64, i64, i64, vp, sz, vp]
        L.gemm_a4w4.restype = i32
        L.grouped_gemm_a4w4_workspace_bytes.argtypes = [ctypes.POINTER(Group), i32, i64, i64]
        L.grouped_gemm_a4w4_workspace_bytes.restype = sz
        L.grouped_gemm_a4w4.argtypes = [ctypes.POINTER(Group), i32, i64, i64, vp, sz, vp]
        L.grouped_gemm_a4w4.restype = i32
        L.grouped_gemm_a4w4_mnk.argtypes = [ctypes.POINTER(GroupMnk), i32, vp]
        L.grouped_gemm_a4w4_mnk.restype = i32
        L.grouped_gemm_nvfp4.argtypes, L.grouped_gemm_nvfp4.restype = [ctypes.POINTER(GroupNv), i32, vp], i32
        _lib = L
        return L


def _check(status: int, where: str) -> None:
    if status != 0:
        raise Mxfp4Error(status, where)


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _require(t: torch.Tensor, dtype: torch.dtype, name: str) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be 2-D with unit column stride")


# Workspace per (device, stream): zeroed once at allocation, grown on demand.
# The library leaves it zeroed after every call, so it is reused without
# clearing. Calls that may overlap need distinct workspaces; calls on one stream
# never overlap, so one buffer per stream is enough. A grown buffer replaces the
# old one only after the stream's earlier work (which may still use the old
# buffer) is ordered before its release by the caching allocator.
_ws: dict = {}


def workspace(device: torch.device, nbytes: int, stream: int | None = None) -> torch.Tensor:
    dev = device.index if device.index is not None else torch.cuda.current_device()
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    key = (dev, int(stream))
    buf = _ws.get(key)
    if nbytes > 0 and (buf is None or buf.numel() < nbytes):
        buf = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=device)
        _ws[key] = buf
    return buf


def quant(x: torch.Tensor, out=None):
    """bf16 [M, K] -> (q uint8 [M, K/2], s uint8 [M, K/32]); `out` = (q, s) reuses given buffers."""
    _require(x, torch.bfloat16, "x")
    M, K = x.shape
    if out is None:
        q = torch.empty((M, K // 2), dtype=torch.uint8, device=x.device)
        s = torch.empty((M, K // 32), dtype=torch.uint8, device=x.device)
    else:
        q, s = out
        _require(q, torch.uint8, "q")
        _require(s, torch.uint8, "s")
        if q.shape != (M, K // 2) or s.shape != (M, K // 32):
            raise ValueError("out buffers must be [M, K/2] and [M, K/32]")
    _check(lib().mxfp4_quant(x.data_ptr(), x.stride(0), q.data_ptr(), q.stride(0), s.data_ptr(), s.stride(0), M, K,
                             _stream(x)), "mxfp4_quant")
    return q, s


def rmsnorm_quant(x: torch.Tensor, w: torch.Tensor, eps: float, out=None):
    """RMSNorm of each row of bf16 x [M, K] with bf16 weight w [K], then MXFP4:
    (q uint8 [M, K/2], s uint8 [M, K/32]); `out` = (q, s) reuses given buffers."""
    _require(x, torch.bfloat16, "x")
    M, K = x.shape
    if not w.is_cuda or w.dtype != torch.bfloat16 or w.dim() != 1 or w.shape[0] != K or w.stride(0) != 1:
        raise ValueError("w must be a contiguous bf16 CUDA vector of length K")
    if out is None:
        q = torch.empty((M, K // 2), dtype=torch.uint8, device=x.device)
        s = torch.empty((M, K // 32), dtype=torch.uint8, device=x.device)
    else:
        q, s = out
        _require(q, torch.uint8, "q")
        _require(s, torch.uint8, "s")
        if q.shape != (M, K // 2) or s.shape != (M, K // 32):
            raise ValueError("out buffers must be [M, K/2] and [M, K/32]")
    _check(lib().mxfp4_rmsnorm_quant(x.data_ptr(), x.stride(0), w.data_ptr(), float(eps), q.data_ptr(), q.stride(0),
                                     s.data_ptr(), s.stride(0), M, K, _stream(x)), "mxfp4_rmsnorm_quant")
    return q, s


def pack_B_bytes(N: int, K: int) -> int:
    return int(lib().mxfp4_pack_B_bytes(N, K))


def pack_B(bq: torch.Tensor, bs: torch.Tensor) -> torch.Tensor:
    """fp4x2 [N, K/2] + E8M0 [N, K/32] (both contiguous uint8) -> packed uint8 buffer."""
    _require(bq, torch.uint8, "bq")
    _require(bs, torch.uint8, "bs")
    N, KH = bq.shape
    K = 2 * KH
    if not (bq.is_contiguous() and bs.is_contiguous()) or bs.shape != (N, K // 32):
        raise ValueError("bq [N, K/2] and bs [N, K/32] must be contiguous and agree")
    out = torch.empty(pack_B_bytes(N, K), dtype=torch.uint8, device=bq.device)
    _check(lib().mxfp4_pack_B(bq.data_ptr(), bs.data_ptr(), N, K, out.data_ptr(), out.numel(), _stream(bq)),
           "mxfp4_pack_B")
    return out


PATHS = {1: "splitk", 2: "skinny", 3: "skinny_tiles", 4: "tiled"}


def fused_path(M: int, N: int, K: int) -> str:
    """Name of the kernel gemm_a4w4_fused runs for (M, N, K) ("splitk", "skinny", "skinny_tiles", "tiled");
    raises for a shape the call rejects."""
    p = int(lib().gemm_a4w4_fused_path(M, N, K))
    if p not in PATHS:
        raise ValueError(f"gemm_a4w4_fused rejects M={M} N={N} K={K}")
    return PATHS[p]


def gemm(a: torch.Tensor, bp: torch.Tensor, N: int, out: torch.Tensor | None = None) -> torch.Tensor:
    """C[M, N] = Q(A) . B^T in one fused launch; A bf16 [M, K], bp from pack_B."""
    _require(a, torch.bfloat16, "a")
    M, K = a.shape
    if bp.numel() < pack_B_bytes(N, K):
        raise ValueError("packed B is smaller than pack_B_bytes(N, K)")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    _require(out, torch.bfloat16, "out")
    wsz = int(lib().gemm_a4w4_workspace_bytes(M, N, K))
    st = _stream(a)
    ws = workspace(a.device, wsz, st)
    _check(lib().gemm_a4w4_fused(a.data_ptr(), a.stride(0), bp.data_ptr(), out.data_ptr(), out.stride(0), M, N, K,
                                 ws.data_ptr() if wsz else None, ws.numel() if wsz else 0, st),
           "gemm_a4w4_fused")
    return out


def gemm_dump(a: torch.Tensor, bp: torch.Tensor, N: int):
    """Verification form of gemm(): returns (C, codes [copies, M, K/2], scales [copies, M, K/32]), the
    quantised A that each N-tile of the fused kernel computed on chip (uint8)."""
    _require(a, torch.bfloat16, "a")
    M, K = a.shape
    if bp.numel() < pack_B_bytes(N, K):
        raise ValueError("packed B is smaller than pack_B_bytes(N, K)")
    out = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    wsz = int(lib().gemm_a4w4_workspace_bytes(M, N, K))
    st = _stream(a)
    ws = workspace(a.device, wsz, st)
    dsz = int(lib().gemm_a4w4_fused_dump_bytes(M, N, K))
    copies = dsz // (M * (K // 2 + K // 32))
    dump = torch.full((dsz,), 0xEE, dtype=torch.uint8, device=a.device)
    _check(lib().gemm_a4w4_fused_dump(a.data_ptr(), a.stride(0), bp.data_ptr(), out.data_ptr(), out.stride(0), M, N, K,
                                      ws.data_ptr() if wsz else None, ws.numel() if wsz else 0, dump.data_ptr(), dsz,
                                      st), "gemm_a4w4_fused_dump")
    nq = copies * M * (K // 2)
    return out, dump[:nq].view(copies, M, K // 2), dump[nq:].view(copies, M, K // 32)


def gemm_a4w4(aq: torch.Tensor, a_scale: torch.Tensor, bp: torch.Tensor, N: int,
              out: torch.Tensor | None = None) -> torch.Tensor:
    """C[M, N] = A_q . B^T with A already quantised: aq fp4x2 [M, K/2], a_scale E8M0 [M, K/32] (uint8,
    for example from quant()); bp from pack_B. The unfused comparator of gemm()."""
    _require(aq, torch.uint8, "aq")
    _require(a_scale, torch.uint8, "a_scale")
    M, KH = aq.shape
    K = 2 * KH
    if a_scale.shape[0] != M or a_scale.shape[1] < K // 32:
        raise ValueError("a_scale must be [M, >= K/32]")
    if bp.numel() < pack_B_bytes(N, K):
        raise ValueError("packed B is smaller than pack_B_bytes(N, K)")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=aq.device)
    _require(out, torch.bfloat16, "out")
    wsz = int(lib().gemm_a4w4_workspace_bytes(M, N, K))
    st = _stream(aq)
    ws = workspace(aq.device, wsz, st)
    _check(lib().gemm_a4w4(aq.data_ptr(), aq.stride(0), a_scale.data_ptr(), a_scale.stride(0), bp.data_ptr(),
                           out.data_ptr(), out.stride(0), M, N, K, ws.data_ptr() if wsz else None,
                           ws.numel() if wsz else 0, st), "gemm_a4w4")
    return out


def grouped_gemm(a_list, bp_list, N: int, out_list=None):
    """One launch over all groups: C_g = Q(A_g) . B_g^T for shared N, K."""
    G = len(a_list)
    if G != len(bp_list):
        raise ValueError("a_list and bp_list differ in length")
    if G < 1 or G > MXFP4_MAX_GROUPS:
        raise ValueError(f"G must be in [1, {MXFP4_MAX_GROUPS}]")
    K = a_list[0].shape[1]
    if out_list is None:
        out_list = [torch.empty((a.shape[0], N), dtype=torch.bfloat16, device=a.device) for a in a_list]
    arr = (Group * G)()
    for g, (a, bp, c) in enumerate(zip(a_list, bp_list, out_list)):
        _require(a, torch.bfloat16, "a_g")
        _require(c, torch.bfloat16, "c_g")
        if a.shape[1] != K:
            raise ValueError("all groups share K")
        arr[g] = Group(a.data_ptr(), a.stride(0), bp.data_ptr(), c.data_ptr(), c.stride(0), a.shape[0])
    wsz = int(lib().grouped_gemm_a4w4_workspace_bytes(arr, G, N, K))
    st = _stream(a_list[0])
    ws = workspace(a_list[0].device, wsz, st)
    _check(lib().grouped_gemm_a4w4(arr, G, N, K, ws.data_ptr() if wsz else None, ws.numel() if wsz else 0, st),
           "grouped_gemm_a4w4")
    return out_list


def grouped_gemm_dump(a_list, bp_list, N: int):
    """Verification form of grouped_gemm(): returns (list of C, list of (codes [copies, M_g, K/2],
    scales [copies, M_g, K/32])), the quantised A each N-tile computed on chip per group."""
    G = len(a_list)
    K = a_list[0].shape[1]
    outs = [torch.empty((a.shape[0], N), dtype=torch.bfloat16, device=a.device) for a in a_list]
    arr = (Group * G)()
    for g, (a, bp, c) in enumerate(zip(a_list, bp_list, outs)):
        _require(a, torch.bfloat16, "a_g")
        arr[g] = Group(a.data_ptr(), a.stride(0), bp.data_ptr(), c.data_ptr(), c.stride(0), a.shape[0])
    dsz = int(lib().grouped_gemm_a4w4_dump_bytes(arr, G, N, K))
    dump = torch.full((dsz,), 0xEE, dtype=torch.uint8, device=a_list[0].device)
    _check(lib().grouped_gemm_a4w4_dump(arr, G, N, K, None, 0, dump.data_ptr(), dsz, _stream(a_list[0])),
           "grouped_gemm_a4w4_dump")
    at, res = 0, []
    for g, a in enumerate(a_list):
        M = a.shape[0]
        copies = int(lib().grouped_gemm_a4w4_dump_copies(arr, G, N, K, g))
        nq, ns = copies * M * (K // 2), copies * M * (K // 32)
        res.append((dump[at:at + nq].view(copies, M, K // 2), dump[at + nq:at + nq + ns].view(copies, M, K // 32)))
        at += nq + ns
    return outs, res


def grouped_gemm_mnk(problems, out_list=None):
    """Groups with their own (M, N, K) and a batch count, in one launch.

    problems: list of (A, Bp, N) with A bf16 [L, M, K] (or [M, K] for L = 1) and
    Bp uint8 [L, pack_B_bytes(N, K)] (or 1-D for L = 1), each batch row-major.
    Returns (or fills `out_list` with) bf16 C tensors [L, M, N] ([M, N] for L = 1).
    """
    descs, outs = [], []
    for gi, (A, Bp, N) in enumerate(problems):
        batched = A.dim() == 3
        A3 = A if batched else A.unsqueeze(0)
        B2 = Bp if Bp.dim() == 2 else Bp.unsqueeze(0)
        L, M, K = A3.shape
        if not A3.is_cuda or A3.dtype != torch.bfloat16 or A3.stride(2) != 1:
            raise ValueError("A must be a bf16 CUDA tensor with unit stride along K")
        if B2.dtype != torch.uint8 or B2.shape[0] != L or B2.shape[1] < pack_B_bytes(N, K) or B2.stride(1) != 1:
            raise ValueError("Bp must be uint8 [L, pack_B_bytes(N, K)]")
        if out_list is None:
            C3 = torch.empty((L, M, N), dtype=torch.bfloat16, device=A.device)
        else:
            C = out_list[gi]
            C3 = C if C.dim() == 3 else C.unsqueeze(0)
            if C3.shape != (L, M, N) or C3.dtype != torch.bfloat16 or C3.stride(2) != 1:
                raise ValueError("out_list[i] must be bf16 [L, M, N]")
        descs.append(GroupMnk(A3.data_ptr(), A3.stride(1), A3.stride(0), B2.data_ptr(), B2.stride(0),
                              C3.data_ptr(), C3.stride(1), C3.stride(0), M, N, K, L))
        outs.append(C3 if batched else C3[0])
    arr = (GroupMnk * len(descs))(*descs)
    _check(lib().grouped_gemm_a4w4_mnk(arr, len(descs), _stream(problems[0][0])), "grouped_gemm_a4w4_mnk")
    return outs if out_list is None else out_list


def grouped_gemm_nvfp4(problems, out_list=None):
    """NVFP4 groups with their own (M, N, K) and a batch count, in one launch.

    problems: list of (aq, a_scale, bq, b_scale): uint8 tensors aq [L, M, K/2]
    (E2M1 codes, low nibble first), a_scale [L, M, K/16] (E4M3), bq [L, N, K/2],
    b_scale [L, N, K/16]; 2-D for L = 1. Rows may be padded (unit stride along
    K). Returns (or fills `out_list` with) float16 C tensors [L, M, N] ([M, N]
    for L = 1).
    """
    def as3(t, name):
        t3 = t if t.dim() == 3 else t.unsqueeze(0)
        if not t3.is_cuda or t3.dtype != torch.uint8 or t3.stride(2) != 1:
            raise ValueError(f"{name} must be a uint8 CUDA tensor with unit stride along K")
        return t3

    descs, outs = [], []
    for gi, (aq, a_s, bq, b_s) in enumerate(problems):
        batched = aq.dim() == 3
        A, As, B, Bs = as3(aq, "aq"), as3(a_s, "a_scale"), as3(bq, "bq"), as3(b_s, "b_scale")
        L, M, KH = A.shape
        N, K = B.shape[1], 2 * KH
        if B.shape != (L, N, KH) or As.shape != (L, M, K // 16) or Bs.shape != (L, N, K // 16):
            raise ValueError("aq [L, M, K/2], a_scale [L, M, K/16], bq [L, N, K/2], b_scale [L, N, K/16] must agree")
        if out_list is None:
            C3 = torch.empty((L, M, N), dtype=torch.float16, device=aq.device)
        else:
            C = out_list[gi]
            C3 = C if C.dim() == 3 else C.unsqueeze(0)
            if C3.shape != (L, M, N) or C3.dtype != torch.float16 or C3.stride(2) != 1:
                raise ValueError("out_list[i] must be float16 [L, M, N]")
        descs.append(GroupNv(A.data_ptr(), A.stride(1), A.stride(0), As.data_ptr(), As.stride(1), As.stride(0),
                             B.data_ptr(), B.stride(1), B.stride(0), Bs.data_ptr(), Bs.stride(1), Bs.stride(0),
                             C3.data_ptr(), C3.stride(1), C3.stride(0), M, N, K, L))
        outs.append(C3 if batched else C3[0])
    arr = (GroupNv * len(descs))(*descs)
    _check(lib().grouped_gemm_nvfp4(arr, len(descs), _stream(problems[0][0])), "grouped_gemm_nvfp4")
    return outs if out_list is None else out_list
