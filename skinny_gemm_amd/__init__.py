"""skinny_gemm_amd -- block-quantized matrix x vector and skinny GEMM
(M = 1..16) for AMD Instinct MI355X (gfx950): Q4_0, Q4_K, Q6_K and IQ4_XS
weights with Q8_1 activations, NVFP4 and FP8 weights with binary16 activations.

The computation lives in libskinny_gemm.so (hand-written HIP kernels behind
the C ABI declared in include/skinny_gemm.h).  This package is its thin
Python binding (same names as the C entry points) plus the build script and
the seeded synthetic input generators.
"""
from ._lib import (  # noqa: F401
    EXPORTS,
    SkinnyError,
    gemv_fp8_w8a16,
    gemv_fp8_w8a16_packed,
    gemv_nvfp4_w4a16,
    gemv_nvfp4_w4a16_packed,
    lib,
    library_path,
    mmvq_iq4_xs,
    mmvq_iq4_xs_packed,
    mmvq_q4_0,
    mmvq_q4_0_f32act,
    mmvq_q4_0_packed,
    mmvq_q4_k,
    mmvq_q4_k_packed,
    mmvq_q6_k,
    mmvq_q6_k_packed,
    prepack_fp8,
    prepack_iq4_xs,
    prepack_iq4_xs_size,
    prepack_fp8_size,
    prepack_nvfp4,
    prepack_q4_0,
    prepack_q4_0_size,
    prepack_q4_k,
    prepack_q4_k_size,
    prepack_q6_k,
    prepack_q6_k_size,
    prepack_nvfp4_size,
    quantize_act_q8_1,
    status_string,
)
