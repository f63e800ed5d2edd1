"""Few-row quantized verify GEMM for MI355X (gfx950): Python binding of libverifygemm.so.

The verify GEMM multiplies M <= 8 drafted activation rows against packed 1-bit sign
(g128) or 2-bit affine (g64) weights, optionally Hadamard-rotated, decoding each weight
once inside the contraction.  All computation runs in the HIP library; this package
only marshals tensors and streams.
"""
from .binding import (  # noqa: F401
    DTYPES, FORMATS, VerifyGemmError, debug_unpack, force_barrier_tail, force_ksplit, force_variant,
    hadamard_rotate, lib, pack_scale_bias, plan_direct, plan_ksplit, plan_variant, release_stream_workspace,
    stream_read, variant_count, variant_name,
    verify_accept_greedy, verify_argmax_rows, verify_gemm, verify_gemm_argmax, verify_gemm_argmax_noalloc,
    verify_gemm_affine1, verify_gemm_affine2, verify_gemm_experts, verify_gemm_had2, verify_gemm_sign1,
)
