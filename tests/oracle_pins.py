"""Pins for the CPU oracle: checks against what the pages and the mathematics fix.

Every function takes the oracle module as ``ref`` and raises AssertionError when a
pin does not hold, so the same checks run against the real oracle (they must pass)
and against copies with a planted mistake (at least one must fail).

Kinds of pin used here:
  * hand-derived closed-form cases stored under tests/golden (exact dyadic values);
  * closed forms on random data (all-ones sign bits give scale * sum(x) per group,
    constant codes give (q*s + b) * sum(x) per group);
  * the Hadamard identities H H^T = n I, involution, Parseval, e0 and ones images,
    and a fast Walsh-Hadamard transform written independently here;
  * invariants: rotating the weights instead of the activations; the MLX 1-bit
    encoding s' = 2s, b' = -s reproducing +-s;
  * brute force with exact rationals (fractions.Fraction) on tiny inputs, with a
    bit-by-bit decoder written independently in pure Python.
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "worked_examples.json")


# ----------------------------------------------------------------------------- helpers
def _f16_fraction(bits: int) -> Fraction:
    """Exact value of an IEEE binary16 bit pattern, decoded field by field."""
    sign = -1 if bits >> 15 else 1
    e = (bits >> 10) & 0x1F
    m = bits & 0x3FF
    if e == 0:
        return sign * Fraction(m, 1 << 24)
    assert e != 31, "inf/nan not expected"
    return sign * Fraction(1024 + m, 1024) * (Fraction(2) ** (e - 15))


def _bf16_fraction(bits: int) -> Fraction:
    sign = -1 if bits >> 15 else 1
    e = (bits >> 7) & 0xFF
    m = bits & 0x7F
    if e == 0:
        return sign * Fraction(m, 128) * (Fraction(2) ** -126)
    return sign * Fraction(128 + m, 128) * (Fraction(2) ** (e - 127))


def _x_spec(spec: str, K: int) -> np.ndarray:
    k = np.arange(K, dtype=np.float64)
    return {"ones": np.ones(K), "iota0": k, "iota1": k + 1.0,
            "e0": (k == 0).astype(np.float64)}[spec]


def _raw_x(x64: np.ndarray, x_dtype: str) -> np.ndarray:
    x64 = np.atleast_2d(x64)
    if x_dtype == "f32":
        return x64.astype(np.float32)
    if x_dtype == "f16":
        return x64.astype(np.float16).view(np.uint16)
    if x_dtype == "bf16":  # the test values used here are exact in bf16 (truncation is exact)
        return (x64.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    raise ValueError(x_dtype)


def _rand_case(rng, fmt, M, K, N, x_dtype="f16"):
    WK = 32 if fmt == "sign1" else 16
    G = 128 if fmt == "sign1" else 64
    words = rng.integers(0, 1 << 32, size=(N, K // WK), dtype=np.uint64).astype(np.uint32)
    s = rng.uniform(0.01, 0.1, size=(N, K // G)).astype(np.float16)
    b = (-rng.uniform(1.0, 2.0, size=s.shape) * s.astype(np.float64)).astype(np.float16)
    x = rng.standard_normal((M, K))
    return words, s.view(np.uint16), b.view(np.uint16), _raw_x(x, x_dtype)


def _close(a, b, rtol=1e-12, atol=1e-12):
    return np.allclose(np.asarray(a, np.float64), np.asarray(b, np.float64), rtol=rtol, atol=atol)


# ----------------------------------------------------------------------------- pins
def pin_decode(ref):
    f16 = {0x3C00: 1.0, 0xC000: -2.0, 0x0001: 2.0 ** -24, 0x7BFF: 65504.0, 0x6400: 1024.0,
           0x0400: 2.0 ** -14, 0x3555: 0.333251953125, 0x8000: -0.0}
    got = ref.decode_f16(np.array(list(f16), dtype=np.uint16))
    assert np.array_equal(got, np.array(list(f16.values()))), got
    bf = {0x3F80: 1.0, 0xC040: -3.0, 0x0001: 2.0 ** -133, 0x7F7F: (2 - 2.0 ** -7) * 2.0 ** 127,
          0x3E80: 0.25, 0xBF00: -0.5}
    got = ref.decode_bf16(np.array(list(bf), dtype=np.uint16))
    assert np.array_equal(got, np.array(list(bf.values()))), got
    x32 = np.array([[1.5, -2.25, 3.0e-8]], dtype=np.float32)
    assert np.array_equal(ref.activations(x32, "f32"), x32.astype(np.float64))


def pin_unpack_hand_words(ref):
    # 1-bit, LSB-first: bit k of word k // 32.
    w = np.array([[0x00000001, 0x80000000, 0xAAAAAAAA, 0x0000FF00]], dtype=np.uint32)
    b = ref.unpack_sign1(w, 128)[0]
    exp = np.zeros(128, dtype=np.uint8)
    exp[0] = 1
    exp[63] = 1
    exp[64:96:2] = 0
    exp[65:96:2] = 1
    exp[96 + 8:96 + 16] = 1
    assert np.array_equal(b, exp), b
    # 2-bit: code k at bits 2(k % 16) of word k // 16.
    w = np.array([[0xE4E4E4E4, 0x00000003, 0xC0000000, 0x0000001B]], dtype=np.uint32)
    q = ref.unpack_affine2(w, 64)[0]
    assert list(q[:16]) == [0, 1, 2, 3] * 4, q[:16]
    assert list(q[16:32]) == [3] + [0] * 15
    assert list(q[32:48]) == [0] * 15 + [3]
    assert list(q[48:52]) == [3, 2, 1, 0] and not q[52:].any()
    assert np.all(ref.unpack_affine2(np.full((1, 4), 0xFFFFFFFF, np.uint32), 64) == 3)
    assert np.all(ref.unpack_sign1(np.full((1, 4), 0xFFFFFFFF, np.uint32), 128) == 1)


def pin_pack_roundtrip(ref):
    rng = np.random.default_rng(11)
    w1 = rng.integers(0, 1 << 32, size=(5, 12), dtype=np.uint64).astype(np.uint32)
    assert np.array_equal(ref.pack_sign1(ref.unpack_sign1(w1, 384)), w1)
    w2 = rng.integers(0, 1 << 32, size=(5, 12), dtype=np.uint64).astype(np.uint32)
    assert np.array_equal(ref.pack_affine2(ref.unpack_affine2(w2, 192)), w2)
    bits = rng.integers(0, 2, size=(3, 256)).astype(np.uint8)
    assert np.array_equal(ref.unpack_sign1(ref.pack_sign1(bits), 256), bits)
    codes = rng.integers(0, 4, size=(3, 128)).astype(np.uint8)
    assert np.array_equal(ref.unpack_affine2(ref.pack_affine2(codes), 128), codes)


def pin_golden(ref):
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    assert len(cases) >= 10
    for c in cases:
        K = c["K"]
        x = _raw_x(_x_spec(c["x"], K), c["x_dtype"])
        words = np.array([[int(h, 16) for h in c["words"]]], dtype=np.uint32)
        s = np.array([[int(h, 16) for h in c["scales"]]], dtype=np.uint16)
        b = None if c["biases"] is None else np.array([[int(h, 16) for h in c["biases"]]], dtype=np.uint16)
        y = ref.verify(c["fmt"], x, c["x_dtype"], words, s, b)
        assert y.shape == (1, 1), (c["name"], y.shape)
        assert _close(y[0, 0], c["y"], rtol=1e-14, atol=1e-14), (c["name"], y[0, 0], c["y"])


def pin_sign1_closed_form(ref):
    """All-ones bits: y[m, n] = sum_g s[n, g] * sum_{k in g} x[m, k]; all-zeros: its negation."""
    rng = np.random.default_rng(3)
    M, K, N = 3, 384, 5
    _, s, _, x = _rand_case(rng, "sign1", M, K, N, "bf16")
    x64 = ref.decode_bf16(x)
    gsum = x64.reshape(M, K // 128, 128).sum(axis=2)                  # [M, G]
    expect = gsum @ s.view(np.float16).astype(np.float64).T           # [M, N]
    ones = np.full((N, K // 32), 0xFFFFFFFF, dtype=np.uint32)
    zeros = np.zeros((N, K // 32), dtype=np.uint32)
    assert _close(ref.verify_sign1(x, "bf16", ones, s), expect)
    assert _close(ref.verify_sign1(x, "bf16", zeros, s), -expect)
    # A bit set in one group only moves that group's term: flip group 1 of row 2 to all ones.
    mixed = zeros.copy()
    mixed[2, 4:8] = 0xFFFFFFFF
    y = ref.verify_sign1(x, "bf16", mixed, s)
    sf = s.view(np.float16).astype(np.float64)
    exp2 = -gsum @ sf[2] + 2 * gsum[:, 1] * sf[2, 1]
    assert _close(y[:, 2], exp2)


def pin_affine2_known_codes(ref):
    """Constant code q: y[m, n] = sum_g (q s[n,g] + b[n,g]) * sum_{k in g} x[m, k]."""
    rng = np.random.default_rng(4)
    M, K, N = 2, 320, 3
    _, s, b, x = _rand_case(rng, "affine2", M, K, N, "f16")
    x64 = ref.decode_f16(x)
    gsum = x64.reshape(M, K // 64, 64).sum(axis=2)
    sf = s.view(np.float16).astype(np.float64)
    bf = b.view(np.float16).astype(np.float64)
    for q, word in ((0, 0x00000000), (1, 0x55555555), (2, 0xAAAAAAAA), (3, 0xFFFFFFFF)):
        words = np.full((N, K // 16), word, dtype=np.uint32)
        expect = gsum @ (q * sf + bf).T
        assert _close(ref.verify_affine2(x, "f16", words, s, b), expect), q
    # dequant of known codes, element by element
    codes = np.array([[0, 1, 2, 3] * 16], dtype=np.uint8)
    w = ref.dequant_affine2(codes, np.array([[0x2800]], np.uint16), np.array([[0xAC00]], np.uint16))
    assert np.array_equal(w[0, :4], [-0.0625, -0.03125, 0.0, 0.03125])


def pin_rowsum_identity(ref):
    """y = sum_g s_g (sum_{k in g} q x) + b_g (sum_{k in g} x): the row-sum form of the affine product."""
    rng = np.random.default_rng(5)
    M, K, N = 4, 256, 7
    words, s, b, x = _rand_case(rng, "affine2", M, K, N, "f16")
    x64 = ref.decode_f16(x)
    q = np.zeros((N, K))
    for n in range(N):
        for k in range(K):
            q[n, k] = (int(words[n, k // 16]) >> (2 * (k % 16))) & 3
    sf = s.view(np.float16).astype(np.float64)
    bf = b.view(np.float16).astype(np.float64)
    qx = np.einsum("mgk,ngk->mng", x64.reshape(M, K // 64, 64), q.reshape(N, K // 64, 64))
    xs = x64.reshape(M, K // 64, 64).sum(axis=2)
    expect = (qx * sf[None]).sum(axis=2) + xs @ bf.T
    assert _close(ref.verify_affine2(x, "f16", words, s, b), expect, rtol=1e-12, atol=1e-12)


def pin_bruteforce_fraction(ref):
    """Exact rational result on tiny inputs; the fp64 oracle must be within its rounding bound."""
    rng = np.random.default_rng(6)
    for fmt, x_dtype, M, K, N in (("sign1", "f32", 2, 256, 3), ("sign1", "bf16", 1, 128, 4),
                                  ("affine2", "f16", 2, 128, 3), ("affine2", "bf16", 2, 64, 2)):
        words, s, b, x = _rand_case(rng, fmt, M, K, N, x_dtype)
        if x_dtype == "f32":
            xf = [[Fraction(float(v)) for v in row] for row in x]
        elif x_dtype == "f16":
            xf = [[_f16_fraction(int(v)) for v in row] for row in x]
        else:
            xf = [[_bf16_fraction(int(v)) for v in row] for row in x]
        y = ref.verify(fmt, x, x_dtype, words, s, None if fmt == "sign1" else b)
        for n in range(N):
            w = []
            for k in range(K):
                if fmt == "sign1":
                    bit = (int(words[n, k // 32]) >> (k % 32)) & 1
                    sc = _f16_fraction(int(s[n, k // 128]))
                    w.append(sc if bit else -sc)
                else:
                    code = (int(words[n, k // 16]) >> (2 * (k % 16))) & 3
                    w.append(code * _f16_fraction(int(s[n, k // 64])) + _f16_fraction(int(b[n, k // 64])))
            for m in range(M):
                exact = sum(xf[m][k] * w[k] for k in range(K))
                bound = K * 2.0 ** -52 * float(sum(abs(xf[m][k] * w[k]) for k in range(K)))
                assert abs(y[m, n] - float(exact)) <= bound + 1e-300, (fmt, m, n, y[m, n], float(exact))


def _fwht(v: np.ndarray) -> np.ndarray:
    """Unnormalized fast Walsh-Hadamard transform along the last axis (butterflies)."""
    v = np.array(v, dtype=np.float64)
    n = v.shape[-1]
    h = 1
    while h < n:
        v = v.reshape(*v.shape[:-1], n // (2 * h), 2, h)
        a, b = v[..., 0, :].copy(), v[..., 1, :].copy()
        v[..., 0, :], v[..., 1, :] = a + b, a - b
        v = v.reshape(*v.shape[:-3], n)
        h *= 2
    return v


def pin_hadamard_identities(ref):
    H = ref.sylvester_hadamard(128)
    assert H.shape == (128, 128)
    assert np.array_equal(H @ H.T, 128 * np.eye(128, dtype=H.dtype))
    i, j = np.meshgrid(np.arange(128), np.arange(128), indexing="ij")
    parity = np.vectorize(lambda a: bin(a).count("1") & 1)(i & j)
    assert np.array_equal(H, 1 - 2 * parity)                     # H[i,j] = (-1)^popcount(i & j)
    Hn = H / math.sqrt(128)
    assert np.allclose(Hn @ Hn, np.eye(128), atol=1e-14)         # symmetric involution
    rng = np.random.default_rng(7)
    x = rng.standard_normal((3, 384))
    xr = ref.hadamard_rotate(x, 128)
    assert np.allclose(np.linalg.norm(xr.reshape(3, 3, 128), axis=2),
                       np.linalg.norm(x.reshape(3, 3, 128), axis=2), rtol=1e-13)
    assert np.allclose(ref.hadamard_rotate(xr, 128), x, atol=1e-13)
    ones = ref.hadamard_rotate(np.ones((1, 128)), 128)[0]
    assert abs(ones[0] - math.sqrt(128)) < 1e-13 and np.abs(ones[1:]).max() < 1e-13
    e0 = np.zeros((1, 256)); e0[0, 128] = 1.0
    r = ref.hadamard_rotate(e0, 128)[0]
    assert np.abs(r[:128]).max() == 0 and np.allclose(r[128:], 1 / math.sqrt(128), rtol=1e-15)
    # the fast transform, written independently, equals the explicit matrix product
    fw = _fwht(x.reshape(3, 3, 128)).reshape(3, 384) / math.sqrt(128)
    assert np.allclose(fw, xr, atol=1e-13)
    assert np.array_equal(ref.sylvester_hadamard(4), np.array([[1, 1, 1, 1], [1, -1, 1, -1],
                                                               [1, 1, -1, -1], [1, -1, -1, 1]]))


def pin_hadamard_blocks_and_signs(ref):
    """Blocks 64 and 256: H H^T = n I, the independent FWHT, the ones image; the signed
    rotation equals the explicit product x D H_bd / sqrt(B), is orthogonal, and undoes to x
    by rotating again and flipping the same signs."""
    rng = np.random.default_rng(17)
    for B in (64, 256):
        H = ref.sylvester_hadamard(B)
        assert np.array_equal(H @ H.T, B * np.eye(B, dtype=H.dtype))
        x = rng.standard_normal((2, 2 * B))
        xr = ref.hadamard_rotate(x, B)
        assert np.allclose(_fwht(x.reshape(2, 2, B)).reshape(2, 2 * B) / math.sqrt(B), xr, atol=1e-13)
        ones = ref.hadamard_rotate(np.ones((1, B)), B)[0]
        assert abs(ones[0] - math.sqrt(B)) < 1e-12 and np.abs(ones[1:]).max() < 1e-12
    K, B = 512, 128
    signs = rng.integers(0, 1 << 32, size=(K // 32,), dtype=np.uint64).astype(np.uint32)
    x = rng.standard_normal((3, K))
    assert np.array_equal(ref.hadamard_rotate(x, B, np.zeros(K // 32, np.uint32)), ref.hadamard_rotate(x, B))
    d = np.array([-1.0 if (int(signs[k // 32]) >> (k % 32)) & 1 else 1.0 for k in range(K)])
    Hbd = np.kron(np.eye(K // B), ref.sylvester_hadamard(B).astype(np.float64)) / math.sqrt(B)
    xs = ref.hadamard_rotate(x, B, signs)
    assert np.allclose(xs, (x * d) @ Hbd, atol=1e-13)
    assert np.allclose(np.linalg.norm(xs, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
    assert np.allclose(ref.hadamard_rotate(xs, B) * d, x, atol=1e-13)
    assert not np.allclose(xs, ref.hadamard_rotate(x, B))


def pin_had2_weight_side(ref):
    """(x Hn) W^T == x (W Hn)^T: rotating the dense weights instead of the activations."""
    rng = np.random.default_rng(8)
    M, K, N = 3, 256, 5
    words, s, b, x = _rand_case(rng, "affine2", M, K, N, "f16")
    y = ref.verify_had2(x, "f16", words, s, b, 128)
    x64 = ref.decode_f16(x)
    w = ref.dequant_affine2(ref.unpack_affine2(words, K), s, b)
    H = ref.sylvester_hadamard(128).astype(np.float64) / math.sqrt(128)
    w_rot = (w.reshape(N, K // 128, 128) @ H).reshape(N, K)
    assert _close(y, x64 @ w_rot.T, rtol=1e-12, atol=1e-12)
    # and the exact rational form: y * sqrt(128) equals x (H_bd) W^T with integer H
    Hi = ref.sylvester_hadamard(128)
    xf = [[_f16_fraction(int(v)) for v in row] for row in x]
    for m in range(M):
        xh = []
        for blk in range(K // 128):
            seg = xf[m][blk * 128:(blk + 1) * 128]
            xh += [sum(seg[i] * int(Hi[i, j]) for i in range(128)) for j in range(128)]
        for n in range(2):
            exact = sum(xh[k] * Fraction(float(w[n, k])) for k in range(K))
            assert abs(y[m, n] * math.sqrt(128) - float(exact)) <= 1e-11 * (1 + abs(float(exact)))


def pin_mlx_1bit_encoding(ref):
    """MLX 1-bit affine encoding s' = 2s, b' = -s with codes {0,1} reproduces +-s exactly."""
    rng = np.random.default_rng(9)
    N, K = 4, 256
    words = rng.integers(0, 1 << 32, size=(N, K // 32), dtype=np.uint64).astype(np.uint32)
    s = rng.uniform(0.01, 0.1, size=(N, K // 128)).astype(np.float16)
    bits = ref.unpack_sign1(words, K)
    w_sign = ref.dequant_sign1(bits, s.view(np.uint16))
    s2 = (2 * s.astype(np.float64)).astype(np.float16)          # exact: doubling an fp16
    bm = (-s.astype(np.float64)).astype(np.float16)
    # expand to the 64-groups of the affine format (each 128-group is two 64-groups)
    s2_64 = np.repeat(s2, 2, axis=1).view(np.uint16)
    bm_64 = np.repeat(bm, 2, axis=1).view(np.uint16)
    w_aff = ref.dequant_affine2(bits, s2_64, bm_64)
    assert np.array_equal(w_sign, w_aff)


def pin_affine1(ref):
    """1-bit affine: the MLX encoding of the sign format reproduces the sign GEMM; all-ones
    and all-zeros bits give the per-group closed forms; exact rational brute force with
    an independent bit decoder."""
    rng = np.random.default_rng(16)
    M, K, N = 3, 384, 5
    words, s, _, x = _rand_case(rng, "sign1", M, K, N, "bf16")
    s64 = s.view(np.float16).astype(np.float64)
    s2 = (2 * s64).astype(np.float16).view(np.uint16)          # exact: doubling an fp16
    bm = (-s64).astype(np.float16).view(np.uint16)
    assert _close(ref.verify_affine1(x, "bf16", words, s2, bm), ref.verify_sign1(x, "bf16", words, s),
                  rtol=1e-13, atol=1e-13)
    b = (-rng.uniform(0.0, 1.0, size=s64.shape) * s64).astype(np.float16).view(np.uint16)
    x64 = ref.decode_bf16(x)
    gsum = x64.reshape(M, K // 128, 128).sum(axis=2)                  # [M, groups]
    sv, bv = ref.decode_f16(s), ref.decode_f16(b)
    ones = np.full_like(words, 0xFFFFFFFF)
    assert _close(ref.verify_affine1(x, "bf16", ones, s, b), gsum @ (sv + bv).T)
    assert _close(ref.verify_affine1(x, "bf16", np.zeros_like(words), s, b), gsum @ bv.T)
    y = ref.verify_affine1(x, "bf16", words, s, b)
    xf = [[_bf16_fraction(int(v)) for v in row] for row in x]
    for n in range(2):
        w = []
        for k in range(K):
            bit = (int(words[n, k // 32]) >> (k % 32)) & 1
            w.append(bit * _f16_fraction(int(s[n, k // 128])) + _f16_fraction(int(b[n, k // 128])))
        for m in range(M):
            exact = sum(xf[m][k] * w[k] for k in range(K))
            bound = K * 2.0 ** -52 * float(sum(abs(xf[m][k] * w[k]) for k in range(K)))
            assert abs(y[m, n] - float(exact)) <= bound + 1e-300, (m, n)


def pin_argmax(ref):
    rng = np.random.default_rng(10)
    M, K, N = 3, 128, 64
    x = rng.standard_normal((M, K)).astype(np.float16)
    star = [7, 40, 63]
    codes = np.zeros((N, K), dtype=np.uint8)
    # planted column star[m]: q = 3 where x[m, k] > 0 and 0 elsewhere, so row m's logit
    # there exceeds every other column's by a wide margin
    for m, nstar in enumerate(star):
        codes[nstar] = np.where(x[m].astype(np.float64) > 0, 3, 0)
    words = ref.pack_affine2(codes)
    s = np.full((N, K // 64), 0x2800, dtype=np.uint16)   # s = 1/32
    b = np.zeros((N, K // 64), dtype=np.uint16)          # b = 0
    y = ref.verify_affine2(x.view(np.uint16), "f16", words, s, b)
    idx, gap = ref.argmax_rows(y)
    assert list(idx) == star, idx
    assert np.all(gap > 0)
    idx, gap = ref.argmax_rows(np.array([[1.0, 3.0, 3.0, 2.0], [5.0, 5.0, 5.0, 5.0]]))
    assert list(idx) == [1, 0] and gap[0] == 0.0 and gap[1] == 0.0


def pin_columns_and_chunks(ref):
    """verify_columns equals a column slice; chunked products equal the one-shot product."""
    rng = np.random.default_rng(12)
    M, K, N = 2, 128, 40
    words, s, b, x = _rand_case(rng, "affine2", M, K, N, "f16")
    y = ref.verify_affine2(x, "f16", words, s, b)
    cols = np.array([0, 5, 39, 17])
    assert _close(ref.verify_columns("affine2", x, "f16", words, s, b, cols), y[:, cols])
    w = ref.dequant_affine2(ref.unpack_affine2(words, K), s, b)
    assert _close(y, ref.decode_f16(x) @ w.T)
    saved = ref.N_CHUNK
    try:
        ref.N_CHUNK = 7
        assert _close(ref.verify_affine2(x, "f16", words, s, b), y)
    finally:
        ref.N_CHUNK = saved


def pin_normwise(ref):
    yr = np.array([[1.0, -4.0, 2.0], [0.5, 0.25, -0.125]])
    yt = yr + np.array([[0.004, 0.0, 0.0], [0.0, -0.001, 0.0]])
    assert abs(ref.normwise_rel_err(yt, yr) - 0.002) < 1e-15
    assert ref.normwise_rel_err(yr, yr) == 0.0


def pin_magnitude(ref):
    """magnitude_columns = sum_k |a_k| |w_k|, by brute force with the independent bit-by-bit
    decoder (and the independent transform for the rotated format); it dominates |y| and
    equals y when every term is non-negative."""
    rng = np.random.default_rng(14)
    for fmt, x_dtype, M, K, N in (("sign1", "bf16", 2, 256, 3), ("affine2", "f16", 2, 128, 3),
                                  ("had2", "f16", 2, 256, 2)):
        words, s, b, x = _rand_case(rng, "sign1" if fmt == "sign1" else "affine2", M, K, N, x_dtype)
        bb = None if fmt == "sign1" else b
        mag = ref.magnitude_columns(fmt, x, x_dtype, words, s, bb)
        y = ref.verify(fmt, x, x_dtype, words, s, bb)
        assert mag.shape == y.shape and np.all(mag >= np.abs(y) * (1 - 1e-12))
        conv = _bf16_fraction if x_dtype == "bf16" else _f16_fraction
        for m in range(M):
            a = [float(conv(int(v))) for v in x[m]]
            if fmt == "had2":
                a = list(_fwht(np.array(a).reshape(K // 128, 128)).reshape(K) / math.sqrt(128))
            for n in range(N):
                tot = 0.0
                for k in range(K):
                    if fmt == "sign1":
                        w = float(_f16_fraction(int(s[n, k // 128])))
                    else:
                        code = (int(words[n, k // 16]) >> (2 * (k % 16))) & 3
                        w = float(code * _f16_fraction(int(s[n, k // 64])) + _f16_fraction(int(b[n, k // 64])))
                    tot += abs(a[k]) * abs(w)
                assert abs(mag[m, n] - tot) <= 1e-12 * tot, (fmt, m, n, mag[m, n], tot)
        cols = np.array([N - 1, 0])
        assert _close(ref.magnitude_columns(fmt, x, x_dtype, words, s, bb, cols), mag[:, cols])
    # all terms non-negative: positive activations, codes, scales and biases
    words, s, b, x = _rand_case(rng, "affine2", 2, 128, 3, "f16")
    x = x & np.uint16(0x7FFF)
    b = s.copy()
    assert _close(ref.magnitude_columns("affine2", x, "f16", words, s, b),
                  ref.verify("affine2", x, "f16", words, s, b), rtol=1e-13, atol=0)


def pin_greedy_accept(ref):
    """Leading-agreement count on planted logits: all rows agree, none agree, the first
    disagreement in the middle, and a disagreement after it that must not count."""
    rng = np.random.default_rng(15)
    y = rng.standard_normal((6, 50))
    top = np.array([3, 17, 17, 0, 49, 8])
    y[np.arange(6), top] = 10.0
    idx, L = ref.greedy_accept(y, top)
    assert list(idx) == list(top) and L == 6
    assert ref.greedy_accept(y, top + 1)[1] == 0
    d = top.copy()
    d[2] = 5
    assert ref.greedy_accept(y, d)[1] == 2
    d[4] = 0
    assert ref.greedy_accept(y, d)[1] == 2
    y[1, 20] = 10.0                      # tie in row 1: the lower index (17) still wins
    assert ref.greedy_accept(y, top)[1] == 6


def pin_experts(ref):
    """Routed-expert verify.  Closed form: expert e holds all-ones sign bits with the exact
    scale (e + 1) / 8, so y[m, s, n] = (route[m, s] + 1) / 8 * sum_k x[m, k]; unused slots
    (route outside 0..E-1) are NaN.  Special case: every slot on one expert reduces to
    the plain product.  Invariant: renumbering the experts (and the route with them)
    changes nothing."""
    E, M, topk, K, N = 4, 3, 3, 256, 5
    words = np.full((E, N, K // 32), 0xFFFFFFFF, dtype=np.uint32)
    scales = np.empty((E, N, K // 128), dtype=np.uint16)
    for e in range(E):
        scales[e] = np.float16((e + 1) / 8).view(np.uint16)
    rng = np.random.default_rng(16)
    x = _raw_x(rng.integers(-8, 9, size=(M, K)).astype(np.float64) / 4, "f16")
    route = np.array([[2, 0, -1], [1, 1, 3], [E, 3, 0]])
    y = ref.verify_experts("sign1", x, "f16", route, words, scales, None)
    assert y.shape == (M, topk, N), y.shape
    xs = ref.decode_f16(x).sum(axis=1)
    for m in range(M):
        for sl in range(topk):
            e = route[m, sl]
            if 0 <= e < E:
                assert np.all(y[m, sl] == (e + 1) / 8 * xs[m]), (m, sl, y[m, sl])
            else:
                assert np.all(np.isnan(y[m, sl])), (m, sl)
    # random weights: one expert everywhere is the plain product; a renumbering is invisible
    fmt = "affine2"
    wr, sr, br = [], [], []
    for e in range(E):
        w1, s1, b1, _ = _rand_case(rng, fmt, 1, K, N)
        wr.append(w1), sr.append(s1), br.append(b1)
    wr, sr, br = np.stack(wr), np.stack(sr), np.stack(br)
    x2 = _raw_x(rng.standard_normal((M, K)), "f16")
    one = ref.verify_experts(fmt, x2, "f16", np.full((M, 2), 2), wr, sr, br)
    plain = ref.verify(fmt, x2, "f16", wr[2], sr[2], br[2])
    assert _close(one[:, 0], plain) and _close(one[:, 1], plain)
    route2 = np.array([[0, 3], [2, 1], [3, 3]])
    perm = np.array([2, 0, 3, 1])                   # new expert i is old expert perm[i]
    inv = np.argsort(perm)
    a = ref.verify_experts(fmt, x2, "f16", route2, wr, sr, br)
    b = ref.verify_experts(fmt, x2, "f16", inv[route2], wr[perm], sr[perm], br[perm])
    assert np.array_equal(a, b)
    cols = np.array([4, 0, 2])
    assert np.array_equal(ref.verify_experts(fmt, x2, "f16", route2, wr, sr, br, rows=cols), a[:, :, cols])


ALL_PINS = [pin_decode, pin_unpack_hand_words, pin_pack_roundtrip, pin_golden,
            pin_sign1_closed_form, pin_affine2_known_codes, pin_rowsum_identity,
            pin_bruteforce_fraction, pin_hadamard_identities, pin_had2_weight_side,
            pin_mlx_1bit_encoding, pin_argmax, pin_columns_and_chunks, pin_normwise,
            pin_magnitude, pin_greedy_accept, pin_affine1, pin_hadamard_blocks_and_signs,
            pin_experts]
