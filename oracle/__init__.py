"""CPU oracle for MXFP4 quantisation and the block-scaled a4w4 GEMM.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package. The product path (the HIP library and its Python binding) never
imports it, and this package imports nothing from the product.

Every function is plain NumPy in float64 (or exact Python integers and
fractions), written from the definitions and unoptimised on purpose.
"""
from .mx import (  # noqa: F401
    E2M1_GRID,
    EMAX_E2M1,
    BLOCK,
    SCALE_BIAS,
    bf16_bits_to_f64,
    f64_to_bf16_bits,
    shared_exponent,
    e2m1_code,
    quant_mx,
    dequant_mx,
    gemm_ref_f64,
    gemm_ref,
    quant_block_exact,
    gemm_exact_fraction,
)
from . import rmsnorm  # noqa: F401,E402  (RMSNorm followed by MXFP4 quantisation)
from . import nvfp4  # noqa: F401,E402  (NVFP4: E2M1 with one E4M3 scale per 16)
