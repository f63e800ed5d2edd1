"""Seeded synthetic inputs shared by the oracle tests, the HIP tests and the benchmark."""
from .inputs import (  # noqa: F401
    GROUP, M_MAX, WORD_K, WORKLOADS, X_DTYPES, Case, bf16_bits, draw_case, draw_signs, draw_x,
    f16_bits,
    workload_case,
)
