"""gemm_a4w4_fused_noalloc (through the C ABI, on an MI355X): the allocation-free
form of gemm_a4w4_fused, whose split-K partials live in a fixed device array
inside the library instead of a caller workspace. Its C must equal
gemm_a4w4_fused's bit for bit (same kernels and arithmetic) and lie within the
oracle's tolerance, on consecutive calls that share the fixed array, the later
ones smaller; and it must leave no state that changes a later call's result."""
import numpy as np
import pytest
import torch

import oracle
from mxfp4_block_scaled_02_amd import ops, synth
from tests.helpers import assert_in_tolerance, bits_of, to_dev_bf16, to_dev_u8

pytestmark = pytest.mark.gpu


def noalloc(a, bp, N):
    M, K = a.shape
    c = torch.full((M, N), 77.0, dtype=torch.bfloat16, device=a.device)
    rc = ops.lib().gemm_a4w4_fused_noalloc(a.data_ptr(), a.stride(0), bp.data_ptr(), c.data_ptr(), c.stride(0), M, N,
                                           K, torch.cuda.current_stream().cuda_stream)
    assert rc == 0, ops.lib().mxfp4_status_str(rc)
    return c


def case(M, N, K, seed):
    g = np.random.default_rng(seed)
    a = synth.f32_to_bf16_bits(g.standard_normal((M, K)).astype(np.float32))
    b = synth.f32_to_bf16_bits((g.standard_normal((N, K)) * 0.02).astype(np.float32))
    bq, bs = oracle.quant_mx(b)
    return a, bq, bs, to_dev_bf16(a), ops.pack_B(to_dev_u8(bq), to_dev_u8(bs))


# The skinny decode shape, then smaller split-K calls (fewer tiles and splits than the first left
# behind in the shared array), then calls that need no scratch (one split; the skinny kernel at M <= 16
# and at 16 < M <= 64; the tiled kernel), then split-K again.
SEQUENCE = [(16, 2112, 7168), (16, 264, 7168), (8, 1000, 6144), (1, 64, 128), (5, 300, 1024), (40, 500, 2048),
            (130, 600, 1024), (16, 2112, 7168)]


def test_noalloc_matches_fused_on_consecutive_calls():
    for i, (M, N, K) in enumerate(SEQUENCE):
        print(f"noalloc call {i}: M={M} N={N} K={K}", flush=True)
        a_bits, bq, bs, a, bp = case(M, N, K, 1000 + i)
        c_ref = ops.gemm(a, bp, N)       # the existing entry point, with its own zeroed workspace
        c = noalloc(a, bp, N)
        torch.cuda.synchronize()
        assert np.array_equal(bits_of(c), bits_of(c_ref)), f"call {i}: differs from gemm_a4w4_fused"
        assert_in_tolerance(bits_of(c), oracle.gemm_ref(a_bits, bq, bs), f"noalloc call {i}")


def test_noalloc_repeated_calls_are_identical():
    a_bits, bq, bs, a, bp = case(16, 2112, 7168, 7)
    outs = [bits_of(noalloc(a, bp, 2112)) for _ in range(5)]
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


def test_noalloc_rejects_geometry_beyond_the_scratch():
    M, N, K = 16, 1088, 65536
    assert ops.lib().gemm_a4w4_workspace_bytes(M, N, K) > (4 << 20)
    a = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    bp = torch.zeros(ops.pack_B_bytes(N, K), dtype=torch.uint8, device="cuda")
    c = torch.full((M, N), 5.0, dtype=torch.bfloat16, device="cuda")
    rc = ops.lib().gemm_a4w4_fused_noalloc(a.data_ptr(), K, bp.data_ptr(), c.data_ptr(), N, M, N, K,
                                           torch.cuda.current_stream().cuda_stream)
    assert rc == 4  # MXFP4_ERR_WORKSPACE, nothing launched
    torch.cuda.synchronize()
    assert (c == 5.0).all()


def test_noalloc_captured_in_a_graph():
    """The callers it is for: a HIP graph captures the call once (no allocation inside the capture) and
    replays it on new data in the same buffers, with eager work in between; every replay must equal the
    eager gemm_a4w4_fused on that data bit for bit (the split-K partials start from zero each time)."""
    M, N, K = 16, 2112, 7168
    _, _, _, a, bp = case(M, N, K, 11)
    c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        rc = ops.lib().gemm_a4w4_fused_noalloc(a.data_ptr(), K, bp.data_ptr(), c.data_ptr(), N, M, N, K,
                                               torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    rng = np.random.default_rng(12)
    for r in range(4):
        print(f"noalloc graph replay {r}", flush=True)
        a.copy_(to_dev_bf16(synth.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))))
        ref = ops.gemm(a, bp, N)      # eager, with its own workspace
        torch.cuda.synchronize()
        c.fill_(3.0)
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits_of(c), bits_of(ref)), f"replay {r} differs from the eager call"
