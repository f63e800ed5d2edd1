"""Seeded synthetic inputs for the few-row verify GEMM.

This module is shared by the CPU oracle's tests and by the HIP path's tests and
benchmark. It holds none of the method's arithmetic: it draws random packed words,
fp16 scales and biases and activation rows, and hands back their raw bit patterns.
Neither the oracle nor the HIP library imports it; the callers pass its arrays on.

Recipe (fixed draw order, one ``numpy.random.default_rng(seed)`` per case):
  1. packed words, uniform over all 32-bit patterns.  A uniform word is exactly
     32 independent uniform sign bits (1-bit format) or 16 independent uniform
     2-bit codes (2-bit format), so no packing step is needed here;
  2. one scale per group, drawn in float64 from U(lo, hi) and rounded to fp16
     (round to nearest even);
  3. formats with biases: one bias per group, drawn using the already rounded scale s
     and then rounded to fp16: U(-2s, -s) for the 2-bit formats (centred codes), U(-s, 0)
     for the 1-bit affine format (weights b and s + b on both sides of zero);
  4. activations: an [8, K] block of N(0, 1) float64 samples, rounded to the
     activation dtype (fp16: nearest even; bf16: first to fp32, then nearest even
     on the fp32 bit pattern; fp32: nearest).  A call with M rows uses the first M
     rows, so sweeps over M share their rows.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

# K-elements per group and per uint32 word for each packed format.
GROUP = {"sign1": 128, "affine2": 64, "had2": 64, "affine1": 128}
WORD_K = {"sign1": 32, "affine2": 16, "had2": 16, "affine1": 32}
SCALE_RANGE = {"sign1": (0.01, 0.1), "affine2": (0.005, 0.05), "had2": (0.005, 0.05),
               "affine1": (0.02, 0.2)}
X_DTYPES = ("f32", "f16", "bf16")
M_MAX = 8

# Named workloads: (format, K, N, activation dtype, row counts exercised).
WORKLOADS = {
    "tiny_sign1_k512_n256": ("sign1", 512, 256, "f32", tuple(range(1, 9))),
    "mlp_up_affine2_k5120_n17408": ("affine2", 5120, 17408, "f16", tuple(range(1, 9))),
    "mlp_up_sign1_k5120_n17408": ("sign1", 5120, 17408, "bf16", tuple(range(1, 9))),
    "mlp_down_sign1_k17408_n5120": ("sign1", 17408, 5120, "bf16", tuple(range(1, 9))),
    "attn_had2_k5120_n6144": ("had2", 5120, 6144, "f16", tuple(range(1, 9))),
    "head_affine2_k5120_n151936": ("affine2", 5120, 151936, "f16", (1, 5, 6, 7, 8)),
    "mlp_up_affine1_k5120_n17408": ("affine1", 5120, 17408, "bf16", tuple(range(1, 9))),
}


def f16_bits(a: np.ndarray) -> np.ndarray:
    """Round float64 values to fp16 (nearest even) and return the uint16 bit patterns."""
    return np.asarray(a, dtype=np.float64).astype(np.float16).view(np.uint16)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float64 values to fp32, then to bf16 (nearest even on the fp32 bits)."""
    u = np.asarray(a, dtype=np.float64).astype(np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


@dataclass
class Case:
    fmt: str
    K: int
    N: int
    x_dtype: str
    words: np.ndarray          # uint32 [N, K / WORD_K]
    scales: np.ndarray         # uint16 fp16 bits [N, K / GROUP]
    biases: np.ndarray | None  # uint16 fp16 bits [N, K / GROUP] (2-bit formats only)
    x_all: np.ndarray          # [8, K]: uint16 bits (f16, bf16) or float32 (f32)

    def x(self, M: int) -> np.ndarray:
        """The first M activation rows, C-contiguous."""
        return np.ascontiguousarray(self.x_all[:M])


def draw_x(rng: np.random.Generator, K: int, x_dtype: str, rows: int = M_MAX) -> np.ndarray:
    z = rng.standard_normal((rows, K))
    if x_dtype == "f16":
        return f16_bits(z)
    if x_dtype == "bf16":
        return bf16_bits(z)
    if x_dtype == "f32":
        return z.astype(np.float32)
    raise ValueError(f"unknown activation dtype {x_dtype!r}")


def draw_case(fmt: str, K: int, N: int, x_dtype: str, seed: int = 0,
              scale_range: tuple[float, float] | None = None) -> Case:
    """Draw one seeded case of a packed format at shape K x N."""
    if fmt not in GROUP:
        raise ValueError(f"unknown format {fmt!r}")
    G, WK = GROUP[fmt], WORD_K[fmt]
    if K % G or K % WK:
        raise ValueError(f"K={K} is not a multiple of the {fmt} group {G}")
    rng = np.random.default_rng(seed)
    words = rng.integers(0, 1 << 32, size=(N, K // WK), dtype=np.uint64).astype(np.uint32)
    lo, hi = scale_range or SCALE_RANGE[fmt]
    s16 = f16_bits(rng.uniform(lo, hi, size=(N, K // G)))
    biases = None
    if fmt in ("affine2", "had2"):
        s = s16.view(np.float16).astype(np.float64)
        biases = f16_bits(rng.uniform(-2.0 * s, -s))
    elif fmt == "affine1":
        s = s16.view(np.float16).astype(np.float64)
        biases = f16_bits(rng.uniform(-s, 0.0))
    x_all = draw_x(rng, K, x_dtype)
    return Case(fmt, K, N, x_dtype, words, s16, biases, x_all)


def workload_case(name: str, seed: int = 0, N: int | None = None) -> Case:
    """Draw a named workload; ``N`` may shrink the output width for quick checks."""
    fmt, K, N0, x_dtype, _ = WORKLOADS[name]
    return draw_case(fmt, K, N0 if N is None else N, x_dtype, seed)


@dataclass
class ExpertsCase:
    fmt: str
    K: int
    N: int
    E: int
    x_dtype: str
    words: np.ndarray          # uint32 [E, N, K / WORD_K]
    scales: np.ndarray         # uint16 fp16 bits [E, N, K / GROUP]
    biases: np.ndarray | None  # uint16 fp16 bits [E, N, K / GROUP]
    x_all: np.ndarray          # [8, K]

    def x(self, M: int) -> np.ndarray:
        return np.ascontiguousarray(self.x_all[:M])


def draw_experts(fmt: str, K: int, N: int, E: int, x_dtype: str, seed: int = 0) -> ExpertsCase:
    """E experts of one layer, each drawn as ``draw_case`` draws one matrix (expert e with
    seed (seed, e)); the activation rows come from expert 0's draw."""
    cases = [draw_case(fmt, K, N, x_dtype, seed=seed * 1000 + e) for e in range(E)]
    biases = None if cases[0].biases is None else np.stack([c.biases for c in cases])
    return ExpertsCase(fmt, K, N, E, x_dtype, np.stack([c.words for c in cases]),
                       np.stack([c.scales for c in cases]), biases, cases[0].x_all)


def draw_route(M: int, topk: int, E: int, seed: int = 0) -> np.ndarray:
    """Router output int32 [M, topk]: each row's topk distinct experts, uniform over the E
    (a mixture-of-experts router picks distinct experts per token)."""
    rng = np.random.default_rng(seed)
    return np.stack([rng.choice(E, size=topk, replace=False) for _ in range(M)]).astype(np.int32)


# Named routed-expert workloads: (format, K, N, E, topk, activation dtype).  The shape is
# a fine-grained mixture-of-experts layer's fused gate and up projection (hidden 2048,
# expert width 768, so N = 2 * 768), 128 experts, 8 routed per token.
EXPERT_WORKLOADS = {
    "moe_gate_up_affine2_e128_top8_k2048_n1536": ("affine2", 2048, 1536, 128, 8, "f16"),
}


def draw_signs(K: int, seed: int = 0) -> np.ndarray:
    """Sign bits of a randomized rotation: uint32 [K/32], each bit uniform (bit set: -1)."""
    rng = np.random.default_rng(seed)
    return rng.integers(0, 1 << 32, size=(K // 32,), dtype=np.uint64).astype(np.uint32)
