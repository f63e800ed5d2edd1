"""CPU fp64 oracle for the few-row quantized verify GEMM (test infrastructure only).

Only the tests, the package smoke check and the benchmark's CPU-baseline leg may
import this package.  The HIP product path never calls it and shares no code with it.
"""
from .verify_ref import (  # noqa: F401
    activations, argmax_rows, greedy_accept, decode_bf16, decode_f16, dequant_affine1, dequant_affine2,
    dequant_sign1,
    hadamard_rotate, magnitude_columns, normwise_rel_err, pack_affine2, pack_sign1, sylvester_hadamard,
    unpack_affine2, unpack_sign1, verify, verify_affine1, verify_affine2, verify_columns, verify_experts, verify_had2,
    verify_sign1,
)
