"""Plant plausible mistakes in a private copy of the oracle; some pin must catch each one.

This checks that the pins are strong enough: a dropped term, a wrong sign, bit order,
index or normalization, or a transposed operand in the oracle has to fail at least
one of them.  Mistakes are planted only in a throwaway copy of the module on the CPU.
"""
import importlib.util
import math

import numpy as np
import pytest

from tests import oracle_pins

REF_PATH = importlib.util.find_spec("oracle.verify_ref").origin


def _fresh_ref():
    spec = importlib.util.spec_from_file_location("oracle_mutant", REF_PATH)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _mut_sign1_msb_first(m):
    def unpack_sign1(words, K):
        w = np.asarray(words, dtype=np.uint32)
        k = np.arange(K)
        return ((w[:, k // 32] >> (31 - k % 32).astype(np.uint32)) & 1).astype(np.uint8)
    m.unpack_sign1 = unpack_sign1


def _mut_affine2_code_order(m):
    def unpack_affine2(words, K):
        w = np.asarray(words, dtype=np.uint32)
        k = np.arange(K)
        return ((w[:, k // 16] >> (2 * (15 - k % 16)).astype(np.uint32)) & 3).astype(np.uint8)
    m.unpack_affine2 = unpack_affine2


def _mut_sign_polarity(m):
    orig = m.dequant_sign1
    m.dequant_sign1 = lambda bits, scales: -orig(bits, scales)


def _mut_drop_bias(m):
    def dequant_affine2(codes, scales, biases):
        K = codes.shape[1]
        g = np.arange(K) // 64
        return codes.astype(np.float64) * m.decode_f16(scales)[:, g]
    m.dequant_affine2 = dequant_affine2


def _mut_sign1_group_size(m):
    def dequant_sign1(bits, scales):
        s = m.decode_f16(scales)
        K = bits.shape[1]
        s_full = s[:, np.minimum(np.arange(K) // 64, s.shape[1] - 1)]
        return np.where(bits.astype(bool), s_full, -s_full)
    m.dequant_sign1 = dequant_sign1


def _mut_affine2_group_index(m):
    def dequant_affine2(codes, scales, biases):
        K = codes.shape[1]
        g = (np.arange(K) % 64) % scales.shape[1]
        return codes.astype(np.float64) * m.decode_f16(scales)[:, g] + m.decode_f16(biases)[:, g]
    m.dequant_affine2 = dequant_affine2


def _signed(x64, signs):
    if signs is None:
        return x64
    k = np.arange(x64.shape[1])
    neg = (np.asarray(signs, dtype=np.uint32)[k // 32] >> (k % 32).astype(np.uint32)) & 1
    return x64 * np.where(neg.astype(bool), -1.0, 1.0)


def _mut_hadamard_unnormalized(m):
    def hadamard_rotate(x64, block=128, signs=None):
        x64 = _signed(x64, signs)
        M, K = x64.shape
        H = m.sylvester_hadamard(block).astype(np.float64)
        return (x64.reshape(M, K // block, block) @ H).reshape(M, K)
    m.hadamard_rotate = hadamard_rotate


def _mut_hadamard_wrong_recursion(m):
    def sylvester_hadamard(n):
        H = np.ones((1, 1), dtype=np.int64)
        while H.shape[0] < n:
            H = np.block([[H, H], [-H, H]])
        return H
    m.sylvester_hadamard = sylvester_hadamard


def _mut_hadamard_skipped(m):
    m.hadamard_rotate = lambda x64, block=128, signs=None: _signed(x64, signs)


def _mut_bf16_shift(m):
    def decode_bf16(bits):
        u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 15
        return u32.view(np.float32).astype(np.float64)
    m.decode_bf16 = decode_bf16


def _mut_f16_as_bf16(m):
    m.decode_f16 = m.decode_bf16


def _mut_rows_reversed(m):
    orig = m.activations
    m.activations = lambda x, dt: orig(x, dt)[::-1]


def _mut_chunk_offset(m):
    def _matmul_chunked(x64, N, dense_rows):
        y = np.empty((x64.shape[0], N))
        for n0 in range(0, N, m.N_CHUNK):
            n1 = min(N, n0 + m.N_CHUNK)
            y[:, n0:n1] = x64 @ dense_rows(0, n1 - n0).T
        return y
    m._matmul_chunked = _matmul_chunked


def _mut_argmax_last_tie(m):
    def argmax_rows(y):
        y = np.asarray(y, dtype=np.float64)
        idx = y.shape[1] - 1 - np.argmax(y[:, ::-1], axis=1)
        s = np.sort(y, axis=1)
        return idx, s[:, -1] - s[:, -2]
    m.argmax_rows = argmax_rows


def _mut_normwise_elementwise(m):
    def normwise_rel_err(a, b):
        a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
        return float(np.max(np.abs(a - b) / np.maximum(np.abs(b), 1e-30)))
    m.normwise_rel_err = normwise_rel_err


def _mut_magnitude_signed_x(m):
    def magnitude_columns(fmt, x, x_dtype, words, scales, biases, cols=None):
        # forgets |a|: the signed activations leak into the bound
        cols = np.arange(words.shape[0]) if cols is None else np.asarray(cols)
        x64 = m.activations(x, x_dtype)
        if fmt == "had2":
            x64 = m.hadamard_rotate(x64, 128)
        K = x64.shape[1]
        if fmt == "sign1":
            w = m.dequant_sign1(m.unpack_sign1(words[cols], K), scales[cols])
        else:
            w = m.dequant_affine2(m.unpack_affine2(words[cols], K), scales[cols], biases[cols])
        return x64 @ np.abs(w).T
    m.magnitude_columns = magnitude_columns


def _mut_magnitude_unrotated(m):
    orig = m.magnitude_columns

    def magnitude_columns(fmt, x, x_dtype, words, scales, biases, cols=None):
        return orig("affine2" if fmt == "had2" else fmt, x, x_dtype, words, scales, biases, cols)
    m.magnitude_columns = magnitude_columns


def _mut_accept_counts_all_matches(m):
    def greedy_accept(y, draft):
        idx, _ = m.argmax_rows(y)
        return idx, int(np.sum(idx == np.asarray(draft).reshape(-1)))
    m.greedy_accept = greedy_accept


def _mut_affine1_group_64(m):
    def dequant_affine1(bits, scales, biases):
        K = bits.shape[1]
        g = np.minimum(np.arange(K) // 64, scales.shape[1] - 1)
        return bits.astype(np.float64) * m.decode_f16(scales)[:, g] + m.decode_f16(biases)[:, g]
    m.dequant_affine1 = dequant_affine1


def _mut_affine1_bias_on_set_bits_only(m):
    def dequant_affine1(bits, scales, biases):
        K = bits.shape[1]
        g = np.arange(K) // 128
        return bits.astype(np.float64) * (m.decode_f16(scales)[:, g] + m.decode_f16(biases)[:, g])
    m.dequant_affine1 = dequant_affine1


def _mut_signs_after_rotation(m):
    orig = m.hadamard_rotate

    def hadamard_rotate(x64, block=128, signs=None):
        y = orig(x64, block)
        if signs is None:
            return y
        k = np.arange(x64.shape[1])
        neg = (np.asarray(signs, dtype=np.uint32)[k // 32] >> (k % 32).astype(np.uint32)) & 1
        return y * np.where(neg.astype(bool), -1.0, 1.0)
    m.hadamard_rotate = hadamard_rotate


def _experts_mutant(m, pick):
    """An explicit routed-expert verify whose (row, slot) -> (x row, expert, output) map
    is `pick(route, m, s, E)` -> (x row, expert or None)."""
    def verify_experts(fmt, x, x_dtype, route, words, scales, biases, rows=None):
        route = np.asarray(route)
        M, topk = route.shape
        E = words.shape[0]
        cols = np.arange(words.shape[1]) if rows is None else np.asarray(rows)
        y = np.full((M, topk, len(cols)), np.nan)
        for r in range(M):
            for sl in range(topk):
                xr, e = pick(route, r, sl, E)
                if e is not None:
                    b = None if biases is None else biases[e]
                    y[r, sl] = m.verify_columns(fmt, x[xr:xr + 1], x_dtype, words[e], scales[e], b, cols)[0]
        return y
    m.verify_experts = verify_experts


def _mut_experts_first_slot_only(m):
    _experts_mutant(m, lambda rt, r, sl, E: (r, int(rt[r, 0]) if 0 <= rt[r, 0] < E else None))


def _mut_experts_slot_as_row(m):
    _experts_mutant(m, lambda rt, r, sl, E: (sl % rt.shape[0], int(rt[r, sl]) if 0 <= rt[r, sl] < E else None))


def _mut_experts_wraps_out_of_range(m):
    _experts_mutant(m, lambda rt, r, sl, E: (r, int(rt[r, sl]) % E))


def _mut_experts_off_by_one(m):
    _experts_mutant(m, lambda rt, r, sl, E: (r, (int(rt[r, sl]) + 1) % E if 0 <= rt[r, sl] < E else None))


MUTATIONS = [_mut_sign1_msb_first, _mut_affine2_code_order, _mut_sign_polarity, _mut_drop_bias,
             _mut_sign1_group_size, _mut_affine2_group_index, _mut_hadamard_unnormalized,
             _mut_hadamard_wrong_recursion, _mut_hadamard_skipped, _mut_bf16_shift,
             _mut_f16_as_bf16, _mut_rows_reversed, _mut_chunk_offset, _mut_argmax_last_tie,
             _mut_normwise_elementwise, _mut_magnitude_signed_x,
             _mut_magnitude_unrotated, _mut_accept_counts_all_matches, _mut_affine1_group_64,
             _mut_affine1_bias_on_set_bits_only, _mut_signs_after_rotation,
             _mut_experts_first_slot_only, _mut_experts_slot_as_row, _mut_experts_wraps_out_of_range,
             _mut_experts_off_by_one]


@pytest.mark.parametrize("mutate", MUTATIONS, ids=lambda f: f.__name__[5:])
def test_planted_mistake_is_caught(mutate):
    mod = _fresh_ref()
    mutate(mod)
    failures = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(mod)
        except (AssertionError, ValueError, IndexError) as exc:  # a pin tripped
            failures.append(pin.__name__)
    assert failures, f"no pin caught the planted mistake {mutate.__name__}"


def test_unmutated_copy_passes_all_pins():
    mod = _fresh_ref()
    for pin in oracle_pins.ALL_PINS:
        pin(mod)
    assert math.isfinite(mod.normwise_rel_err(np.ones((1, 2)), np.ones((1, 2))))
