"""Seeded synthetic inputs shared by the oracle tests, the HIP tests and the benchmark."""
from .inputs import (  # noqa: F401
    EXPERT_WORKLOADS, GROUP, M_MAX, WORD_K, WORKLOADS, X_DTYPES, Case, ExpertsCase, bf16_bits,
    draw_case, draw_experts, draw_route, draw_signs, draw_x, f16_bits, workload_case,
)
