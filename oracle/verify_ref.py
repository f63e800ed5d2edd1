"""CPU fp64 oracle for the few-row quantized verify GEMM.

TEST INFRASTRUCTURE.  Only the tests, the package's smoke check and the benchmark's
CPU-baseline leg may import or run this module.  The HIP library never calls it, and
the two share no code: no kernels, helpers, tables or pre/post-processing.

What the method computes.  Speculative decoding checks a block of M drafted rows in
one pass; the verify kernel decodes each packed weight once and multiplies it
against every drafted row ("Ishizuki" README, "Kernels written for the verify";
"dflash-mlx-bonsai2" README, "Why").  Up to summation order the result is the plain
product  y[m, n] = sum_k x[m, k] * w[n, k]  of the activations with the dequantized
weights, so this oracle is that definition written out in float64 numpy: unpack,
dequantize, (rotate,) multiply.  Every fp16, bf16 and fp32 input is exactly
representable in float64, so the only rounding is numpy's fp64 summation.

Formats:
  sign1  -- one sign bit per weight, bit 0 -> -scale, bit 1 -> +scale, one fp16
            scale per 128 consecutive weights of an output row ("Bonsai-27B-mlx-1bit"
            model card, the paragraph on the binary weight format).
  affine2 -- 2-bit code q in {0,1,2,3}, w = q*s + b with one fp16 scale s and one
            fp16 bias b per 64 consecutive weights (MLX's grouped affine format,
            which stores a scale and a bias per group: same model card, MLX paragraph;
            "Ishizuki" README, MLX affine codes).
  affine1 -- MLX's 1-bit affine codes: one bit c per weight, w = c*s + b with one fp16
            scale and one fp16 bias per 128 consecutive weights; the sign format is the
            case s = 2*s_sign, b = -s_sign ("Bonsai-27B-mlx-1bit" model card, MLX
            paragraph).  Bits are packed exactly like the sign bits.
  had2   -- the 2-bit affine format applied to activations first multiplied by a
            block-diagonal normalized Sylvester Hadamard matrix with block 128
            ("dflash-mlx-bonsai2" README, "What this fork adds": Hadamard-rotated 2-bit
            pack, verify prep with a fused Hadamard; "Ishizuki" README: the rotation
            is declared by the pack).

Readings taken where the pages are silent:
  * bit order: LSB-first within little-endian uint32 words.  Weight k of a 1-bit row
    is bit k%32 of word k//32; code k of a 2-bit row sits at bits 2*(k%16)..+1 of
    word k//16.  Groups start at k = 0.
  * scales and biases are separate fp16 arrays of shape [N, K/G], row-major.
  * the output is fp32 [M, N] on the GPU; the oracle returns fp64.
  * the Hadamard step is x' = x @ H_bd with H_bd block-diagonal, each block
    H_128 / sqrt(128) built by the Sylvester recursion; no random sign diagonal.
  * argmax ties go to the lowest column index.
"""
from __future__ import annotations

import numpy as np

N_CHUNK = 16384  # output columns dequantized at a time (bounds the dense fp64 block)


# ----------------------------------------------------------------------------- decoding
def decode_f16(bits: np.ndarray) -> np.ndarray:
    """IEEE binary16 bit patterns -> float64 (exact)."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float64 (exact): bf16 is the upper half of an fp32."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u32.view(np.float32).astype(np.float64)


def activations(x: np.ndarray, x_dtype: str) -> np.ndarray:
    """Raw activation rows (uint16 bits for f16/bf16, float32 for f32) -> float64."""
    if x_dtype == "f16":
        return decode_f16(x)
    if x_dtype == "bf16":
        return decode_bf16(x)
    if x_dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    raise ValueError(f"unknown activation dtype {x_dtype!r}")


# ----------------------------------------------------------------------------- unpacking
def unpack_sign1(words: np.ndarray, K: int) -> np.ndarray:
    """uint32 [N, K/32] -> bits uint8 [N, K]; bit k is (word[k // 32] >> (k % 32)) & 1."""
    w = np.asarray(words, dtype=np.uint32)
    k = np.arange(K)
    return ((w[:, k // 32] >> (k % 32).astype(np.uint32)) & 1).astype(np.uint8)


def unpack_affine2(words: np.ndarray, K: int) -> np.ndarray:
    """uint32 [N, K/16] -> codes uint8 [N, K]; code k is (word[k // 16] >> 2*(k % 16)) & 3."""
    w = np.asarray(words, dtype=np.uint32)
    k = np.arange(K)
    return ((w[:, k // 16] >> (2 * (k % 16)).astype(np.uint32)) & 3).astype(np.uint8)


def pack_sign1(bits: np.ndarray) -> np.ndarray:
    """Inverse of unpack_sign1 (used to build hand-made cases and round-trip checks)."""
    b = np.asarray(bits, dtype=np.uint64)
    N, K = b.shape
    out = np.zeros((N, K // 32), dtype=np.uint64)
    for j in range(32):
        out |= b[:, j::32] << np.uint64(j)
    return out.astype(np.uint32)


def pack_affine2(codes: np.ndarray) -> np.ndarray:
    """Inverse of unpack_affine2."""
    q = np.asarray(codes, dtype=np.uint64)
    N, K = q.shape
    out = np.zeros((N, K // 16), dtype=np.uint64)
    for j in range(16):
        out |= (q[:, j::16] & np.uint64(3)) << np.uint64(2 * j)
    return out.astype(np.uint32)


# ----------------------------------------------------------------------------- dequant
def dequant_sign1(bits: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """w[n, k] = +s[n, k // 128] if bit else -s[n, k // 128]   (fp64)."""
    s = decode_f16(scales)
    K = bits.shape[1]
    s_full = s[:, np.arange(K) // 128]
    return np.where(bits.astype(bool), s_full, -s_full)


def dequant_affine2(codes: np.ndarray, scales: np.ndarray, biases: np.ndarray) -> np.ndarray:
    """w[n, k] = q[n, k] * s[n, k // 64] + b[n, k // 64]   (fp64, exact for fp16 s, b)."""
    K = codes.shape[1]
    g = np.arange(K) // 64
    return codes.astype(np.float64) * decode_f16(scales)[:, g] + decode_f16(biases)[:, g]


def dequant_affine1(bits: np.ndarray, scales: np.ndarray, biases: np.ndarray) -> np.ndarray:
    """w[n, k] = bit[n, k] * s[n, k // 128] + b[n, k // 128]   (fp64, exact for fp16 s, b)."""
    K = bits.shape[1]
    g = np.arange(K) // 128
    return bits.astype(np.float64) * decode_f16(scales)[:, g] + decode_f16(biases)[:, g]


# ----------------------------------------------------------------------------- Hadamard
def sylvester_hadamard(n: int) -> np.ndarray:
    """H_1 = [1],  H_2m = [[H_m, H_m], [H_m, -H_m]]  (integer matrix, n a power of two)."""
    if n < 1 or n & (n - 1):
        raise ValueError("Hadamard order must be a power of two")
    H = np.ones((1, 1), dtype=np.int64)
    while H.shape[0] < n:
        H = np.block([[H, H], [H, -H]])
    return H


def hadamard_rotate(x64: np.ndarray, block: int = 128, signs: np.ndarray | None = None) -> np.ndarray:
    """x' = (x D) @ blockdiag(H_block / sqrt(block)), applied to each aligned block of K, with
    D = diag(d_k), d_k = -1 where bit k % 32 of signs[k // 32] is set (D = I if signs is None).
    The sign step is the plainest reading of the "sign" in the fused prep of the
    "dflash-mlx-bonsai2" README ("What this fork adds"): a diagonal of +-1 before the
    rotation."""
    M, K = x64.shape
    if K % block:
        raise ValueError("K must be a multiple of the Hadamard block")
    if signs is not None:
        k = np.arange(K)
        neg = (np.asarray(signs, dtype=np.uint32)[k // 32] >> (k % 32).astype(np.uint32)) & 1
        x64 = x64 * np.where(neg.astype(bool), -1.0, 1.0)
    Hn = sylvester_hadamard(block).astype(np.float64) / np.sqrt(float(block))
    return (x64.reshape(M, K // block, block) @ Hn).reshape(M, K)


# ----------------------------------------------------------------------------- verify GEMMs
def _matmul_chunked(x64: np.ndarray, N: int, dense_rows) -> np.ndarray:
    y = np.empty((x64.shape[0], N), dtype=np.float64)
    for n0 in range(0, N, N_CHUNK):
        n1 = min(N, n0 + N_CHUNK)
        y[:, n0:n1] = x64 @ dense_rows(n0, n1).T
    return y


def verify_sign1(x: np.ndarray, x_dtype: str, words: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """y[M, N] = x[M, K] @ W^T with W the dequantized 1-bit sign weights (fp64)."""
    x64 = activations(x, x_dtype)
    K = x64.shape[1]
    return _matmul_chunked(x64, words.shape[0],
                           lambda a, b: dequant_sign1(unpack_sign1(words[a:b], K), scales[a:b]))


def verify_affine2(x: np.ndarray, x_dtype: str, words: np.ndarray, scales: np.ndarray,
                   biases: np.ndarray) -> np.ndarray:
    """y[M, N] = x[M, K] @ W^T with W the dequantized 2-bit affine weights (fp64)."""
    x64 = activations(x, x_dtype)
    K = x64.shape[1]
    return _matmul_chunked(x64, words.shape[0],
                           lambda a, b: dequant_affine2(unpack_affine2(words[a:b], K),
                                                        scales[a:b], biases[a:b]))


def verify_affine1(x: np.ndarray, x_dtype: str, words: np.ndarray, scales: np.ndarray,
                   biases: np.ndarray) -> np.ndarray:
    """y[M, N] = x[M, K] @ W^T with W the dequantized 1-bit affine weights (fp64)."""
    x64 = activations(x, x_dtype)
    K = x64.shape[1]
    return _matmul_chunked(x64, words.shape[0],
                           lambda a, b: dequant_affine1(unpack_sign1(words[a:b], K),
                                                        scales[a:b], biases[a:b]))


def verify_had2(x: np.ndarray, x_dtype: str, words: np.ndarray, scales: np.ndarray,
                biases: np.ndarray, block: int = 128, signs: np.ndarray | None = None) -> np.ndarray:
    """Unfused reference: rotate the activations (optionally sign-flipped first), then the
    2-bit affine product."""
    x64 = hadamard_rotate(activations(x, x_dtype), block, signs)
    K = x64.shape[1]
    return _matmul_chunked(x64, words.shape[0],
                           lambda a, b: dequant_affine2(unpack_affine2(words[a:b], K),
                                                        scales[a:b], biases[a:b]))


def verify_columns(fmt: str, x: np.ndarray, x_dtype: str, words: np.ndarray,
                   scales: np.ndarray, biases: np.ndarray | None, cols: np.ndarray,
                   block: int = 128, signs: np.ndarray | None = None) -> np.ndarray:
    """The oracle restricted to a sample of output columns: y[:, cols] (block and signs:
    the rotation of the had2 format)."""
    cols = np.asarray(cols)
    w = words[cols]
    s = scales[cols]
    b = None if biases is None else biases[cols]
    if fmt == "sign1":
        return verify_sign1(x, x_dtype, w, s)
    if fmt == "affine2":
        return verify_affine2(x, x_dtype, w, s, b)
    if fmt == "had2":
        return verify_had2(x, x_dtype, w, s, b, block, signs)
    if fmt == "affine1":
        return verify_affine1(x, x_dtype, w, s, b)
    raise ValueError(f"unknown format {fmt!r}")


def verify(fmt: str, x, x_dtype, words, scales, biases=None) -> np.ndarray:
    if fmt == "sign1":
        return verify_sign1(x, x_dtype, words, scales)
    if fmt == "affine2":
        return verify_affine2(x, x_dtype, words, scales, biases)
    if fmt == "had2":
        return verify_had2(x, x_dtype, words, scales, biases)
    if fmt == "affine1":
        return verify_affine1(x, x_dtype, words, scales, biases)
    raise ValueError(f"unknown format {fmt!r}")


def magnitude_columns(fmt: str, x: np.ndarray, x_dtype: str, words: np.ndarray,
                      scales: np.ndarray, biases: np.ndarray | None, cols=None,
                      block: int = 128, signs: np.ndarray | None = None) -> np.ndarray:
    """mag[m, n] = sum_k |a[m, k]| * |w[n, k]|, the sum of the magnitudes of the terms of
    y[m, n] (a = the activations, rotated for had2; w = the dequantized weights), for the
    columns `cols` (all if None).  Bounds how far any summation order and any rounding of
    the individual terms can move y: a relative rounding u of each term moves y by at
    most u * mag."""
    cols = np.arange(words.shape[0]) if cols is None else np.asarray(cols)
    x64 = activations(x, x_dtype)
    if fmt == "had2":
        x64 = hadamard_rotate(x64, block, signs)
    K = x64.shape[1]
    w, s = words[cols], scales[cols]
    if fmt == "sign1":
        dense = lambda a, b: dequant_sign1(unpack_sign1(w[a:b], K), s[a:b])
    elif fmt == "affine1":
        b1 = biases[cols]
        dense = lambda a, b: dequant_affine1(unpack_sign1(w[a:b], K), s[a:b], b1[a:b])
    elif fmt in ("affine2", "had2"):
        bb = biases[cols]
        dense = lambda a, b: dequant_affine2(unpack_affine2(w[a:b], K), s[a:b], bb[a:b])
    else:
        raise ValueError(f"unknown format {fmt!r}")
    return _matmul_chunked(np.abs(x64), len(cols), lambda a, b: np.abs(dense(a, b)))


def verify_experts(fmt: str, x: np.ndarray, x_dtype: str, route: np.ndarray, words: np.ndarray,
                   scales: np.ndarray, biases: np.ndarray | None, rows=None) -> np.ndarray:
    """Routed-expert verify ("Ijah" README, "What's new (v0.2)": rows verified together
    are routed to experts, and each expert's weights serve every row routed to it).

    route int [M, topk]: the expert of each (row, slot), a value outside 0..E-1 marking an
    unused slot; words, scales, biases: the E experts' packed weights stacked on axis 0.
    Returns y[M, topk, N] (or only the output columns `rows`) with
    y[m, s] = x[m] @ W_route[m, s]^T in fp64 and NaN in unused slots.  Grouping the rows
    by expert changes which rows share a weight read, not what any row computes, so this
    is the per-(row, slot) product of the format written out."""
    route = np.asarray(route)
    M, topk = route.shape
    E = words.shape[0]
    cols = np.arange(words.shape[1]) if rows is None else np.asarray(rows)
    y = np.full((M, topk, len(cols)), np.nan)
    for m in range(M):
        for s in range(topk):
            e = int(route[m, s])
            if 0 <= e < E:
                b = None if biases is None else biases[e]
                y[m, s] = verify_columns(fmt, x[m:m + 1], x_dtype, words[e], scales[e], b, cols)[0]
    return y


# ----------------------------------------------------------------------------- head + checks
def argmax_rows(y: np.ndarray):
    """Per-row argmax (first index on ties) and the gap between the top two values."""
    y = np.asarray(y, dtype=np.float64)
    idx = np.argmax(y, axis=1)
    top2 = np.sort(y, axis=1)[:, -2:] if y.shape[1] > 1 else np.concatenate([y, y], axis=1)
    return idx.astype(np.int64), top2[:, 1] - top2[:, 0]


def greedy_accept(y: np.ndarray, draft: np.ndarray):
    """Greedy acceptance of a drafted block ("dflash-mlx-bonsai2" README, "Verify it
    yourself": the verify keeps the drafted tokens the target's argmax agrees with).
    Returns (argmax per row, L) with L the number of leading rows m whose argmax equals
    draft[m]."""
    idx, _ = argmax_rows(y)
    draft = np.asarray(draft).reshape(-1)
    L = 0
    while L < len(idx) and idx[L] == draft[L]:
        L += 1
    return idx, L


def normwise_rel_err(y_test: np.ndarray, y_ref: np.ndarray) -> float:
    """max over rows m of  max_n |y_test - y_ref| / max_n |y_ref|."""
    y_test = np.asarray(y_test, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    num = np.max(np.abs(y_test - y_ref), axis=1)
    den = np.max(np.abs(y_ref), axis=1)
    den = np.where(den > 0, den, 1.0)
    return float(np.max(num / den)) if num.size else 0.0
