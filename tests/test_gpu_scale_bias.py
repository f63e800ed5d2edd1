"""GPU parity of the interleaved scale-and-bias layout of the affine formats.

vg_pack_scale_bias must move every value bit for bit, and a verify call given the
interleaved pairs (biases NULL) must return what the same call on the two separate arrays
returns, bit for bit (the same values reach the same arithmetic), and what the fp64 oracle
computes, to the bar of the plain calls.  The pairs are the MLX grouped affine format's own
scale and bias per group ("Bonsai-27B-mlx-1bit" model card, MLX paragraph), stored side by
side.
"""
import json
import os

import numpy as np
import pytest

from synthetic import draw_case, draw_experts, draw_route, draw_signs
from synthetic.torch_io import case_tensors, f16_tensor
from tests.test_gpu_parity import GOLDEN, check, workload_ref

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

Q, H, VALU, GEMV = 0, 1, 2, 3


@pytest.fixture(scope="module")
def vg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import few_row_quantized_verify_amd as m
    m.lib()  # fails loudly if the library is missing
    m.force_variant(-1)
    m.force_ksplit(0)
    yield m
    m.force_variant(-1)
    m.force_ksplit(0)


def both(vg, case, M, call):
    """call(x, w, scales, biases) on the separate arrays, then on the pairs packed on the
    device; returns the two outputs as float64 arrays."""
    x, w, s, b = case_tensors(case, M)
    sb = vg.pack_scale_bias(s, b)
    y_sep = call(x, w, s, b)
    y_sbi = call(x, w, sb, None)
    torch.cuda.synchronize()
    return y_sep.cpu().numpy().astype(np.float64), y_sbi.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("shape", [(1,), (255,), (256,), (257,), (100003,), (3, 17, 40)])
def test_pack_moves_every_value(vg, shape):
    """Random 16-bit patterns (NaN and infinity patterns included): the packed array holds
    each scale and its bias side by side, unchanged."""
    rng = np.random.default_rng(sum(shape))
    s = rng.integers(0, 1 << 16, size=shape, dtype=np.uint32).astype(np.uint16)
    b = rng.integers(0, 1 << 16, size=shape, dtype=np.uint32).astype(np.uint16)
    out = vg.pack_scale_bias(f16_tensor(s, "cuda"), f16_tensor(b, "cuda"))
    torch.cuda.synchronize()
    got = out.cpu().view(torch.int16).numpy().view(np.uint16)
    assert got.shape == (*shape, 2)
    assert np.array_equal(got[..., 0], s) and np.array_equal(got[..., 1], b)


def test_pack_zero_count_enqueues_nothing(vg):
    buf = torch.full((64,), 3.0, dtype=torch.float16, device="cuda")
    L = vg.lib()
    assert L.vg_pack_scale_bias(buf.data_ptr(), buf.data_ptr(), 0, buf.data_ptr(), None) == 0
    torch.cuda.synchronize()
    assert torch.all(buf == 3.0)


CASES = [("affine2", 3072, 100), ("had2", 2048, 100), ("affine1", 2048, 100)]


@pytest.mark.parametrize("fmt,K,N", CASES)
@pytest.mark.parametrize("x_dtype", ["f16", "bf16", "f32"])
def test_every_variant_matches_separate_arrays(vg, fmt, K, N, x_dtype):
    """Every kernel variant that takes the call (the two MFMA row-block modes, the dot2
    kernel, the fp32 VALU kernel), every row count it takes, several tiles and a ragged last
    one: bit-identical to the separate arrays, and within the oracle's bounds."""
    case = draw_case(fmt, K, N, x_dtype, seed=31)
    ran = set()
    try:
        for v in (Q, H, GEMV, VALU):
            vg.force_variant(v)
            for M in range(1, 9):
                if vg.plan_variant(fmt, x_dtype, M, N, K) < 0:
                    continue
                y_sep, y_sbi = both(vg, case, M, lambda x, w, s, b: vg.verify_gemm(fmt, x, w, s, b))
                assert np.array_equal(y_sep, y_sbi), (vg.variant_name(v), M)
                check(case, M, y_sbi, label=f"sbi[{vg.variant_name(v)}]")
                ran.add(v)
    finally:
        vg.force_variant(-1)
    assert ran == ({VALU} if x_dtype == "f32" else {Q, H, GEMV, VALU}), ran


@pytest.mark.parametrize("block", [64, 256])
def test_signed_rotation(vg, block):
    case = draw_case("had2", 2048, 77, "f16", seed=32)
    signs = torch.from_numpy(draw_signs(2048, seed=5).view(np.int32)).cuda()
    for M in (1, 4, 8):
        y_sep, y_sbi = both(vg, case, M, lambda x, w, s, b: vg.verify_gemm_had2(x, w, s, b, had_block=block,
                                                                               signs=signs))
        assert np.array_equal(y_sep, y_sbi), M


@pytest.mark.parametrize("name", ["mlp_up_affine2_k5120_n17408", "attn_had2_k5120_n6144",
                                  "mlp_up_affine1_k5120_n17408"])
def test_full_workload_every_row_count(vg, name):
    """The full-size affine workloads at every row count, every column, in the launch
    configuration the benchmark times: against the oracle, and bit-identical to the
    separate arrays."""
    case, ref = workload_ref(name)
    for M in range(1, 9):
        y_sep, y_sbi = both(vg, case, M, lambda x, w, s, b: vg.verify_gemm(case.fmt, x, w, s, b))
        assert np.array_equal(y_sep, y_sbi), M
        check(case, M, y_sbi, ref=ref, label=f"{name}[sbi]")


def test_head_argmax(vg):
    """The output head through the fused-argmax call: each row's argmax equal to the
    oracle's stored one, the logits bit-identical to the separate arrays' and, at M = 1
    and 8, every logit within the oracle's bounds."""
    with open(os.path.join(GOLDEN, "head_affine2_k5120_n151936_argmax.json")) as f:
        gold = json.load(f)
    case, ref = workload_ref(gold["workload"])
    for M in (1, 5, 6, 7, 8):
        x, w, s, b = case_tensors(case, M)
        sb = vg.pack_scale_bias(s, b)
        y_sep, i_sep = vg.verify_gemm_argmax("affine2", x, w, s, b)
        y_sbi, i_sbi = vg.verify_gemm_argmax("affine2", x, w, sb, None)
        assert torch.equal(y_sep, y_sbi) and torch.equal(i_sep, i_sbi), M
        assert i_sbi.cpu().tolist() == gold["argmax"][:M], M
        if M in (1, 8):
            check(case, M, y_sbi.cpu().numpy().astype(np.float64), ref=ref, label="head[sbi]")


def test_forced_k_split(vg):
    """K split across workgroups (partials reduced by the last slice) with the pairs."""
    case = draw_case("affine2", 4096, 300, "f16", seed=33)
    try:
        for ks in (2, 4):
            vg.force_ksplit(ks)
            for M in (2, 7):
                y_sep, y_sbi = both(vg, case, M, lambda x, w, s, b: vg.verify_gemm("affine2", x, w, s, b))
                assert np.array_equal(y_sep, y_sbi), (ks, M)
                check(case, M, y_sbi, label=f"sbi-ks{ks}")
    finally:
        vg.force_ksplit(0)


@pytest.mark.parametrize("fmt", ["affine2", "had2", "affine1"])
@pytest.mark.parametrize("M", [3, 8])
def test_grouped_experts(vg, fmt, M):
    """The grouped routed-expert verify with stacked interleaved pairs [E, N, K/G, 2]."""
    E, topk = 6, 3
    ec = draw_experts(fmt, 2048, 200, E, "f16", seed=34)
    route = torch.from_numpy(draw_route(M, topk, E, seed=M)).cuda()
    x, w, s, b = case_tensors(ec, M)
    sb = vg.pack_scale_bias(s, b)
    y_sep = torch.zeros((M, topk, ec.N), dtype=torch.float32, device="cuda")
    y_sbi = torch.ones((M, topk, ec.N), dtype=torch.float32, device="cuda")
    vg.verify_gemm_experts(fmt, x, route, w, s, b, y=y_sep)
    vg.verify_gemm_experts(fmt, x, route, w, sb, None, y=y_sbi)
    torch.cuda.synchronize()
    assert torch.equal(y_sep, y_sbi)


def test_no_alloc_entry_point(vg):
    case = draw_case("affine2", 2048, 333, "f16", seed=35)
    for M in (1, 6):
        x, w, s, b = case_tensors(case, M)
        sb = vg.pack_scale_bias(s, b)
        idx = torch.empty((M,), dtype=torch.int32, device="cuda")
        y_ref, i_ref = vg.verify_gemm_argmax("affine2", x, w, s, b)
        y = torch.empty_like(y_ref)
        vg.verify_gemm_argmax_noalloc("affine2", x, w, sb, None, y, idx=idx)
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref) and torch.equal(idx, i_ref), M


def test_pairs_of_another_draw_change_the_output(vg):
    """A bar on the comparison itself: the interleaved pairs are read (another draw's pairs
    change the output)."""
    c1 = draw_case("affine2", 1024, 64, "f16", seed=36)
    c2 = draw_case("affine2", 1024, 64, "f16", seed=37)
    x, w, s, b = case_tensors(c1, 2)
    sb2 = vg.pack_scale_bias(f16_tensor(c2.scales, "cuda"), f16_tensor(c2.biases, "cuda"))
    y1 = vg.verify_gemm("affine2", x, w, s, b)
    y2 = vg.verify_gemm("affine2", x, w, sb2, None)
    torch.cuda.synchronize()
    assert not torch.equal(y1, y2)


@pytest.mark.parametrize("fmt,x_dtype", [("affine2", "f16"), ("had2", "bf16"), ("affine1", "f16")])
def test_long_k_several_windows(vg, fmt, x_dtype):
    """K = 16384 in one slice (forced), so each workgroup stages its activations in several LDS
    windows and the pairs' offsets move with the window."""
    case = draw_case(fmt, 16384, 300, x_dtype, seed=38)
    try:
        vg.force_ksplit(1)
        for M in (2, 8):
            y_sep, y_sbi = both(vg, case, M, lambda x, w, s, b: vg.verify_gemm(fmt, x, w, s, b))
            assert np.array_equal(y_sep, y_sbi), M
            check(case, M, y_sbi, label="sbi-long-k")
    finally:
        vg.force_ksplit(0)


@pytest.mark.parametrize("fmt,K", [("affine2", 4160), ("had2", 4224), ("affine1", 2176)])
@pytest.mark.parametrize("x_dtype", ["f32", "f16"])
def test_valu_windows(vg, fmt, K, x_dtype):
    """K not a multiple of 1024: the VALU kernel, its activation windows and a narrow last one,
    reading each group's pair as one word."""
    case = draw_case(fmt, K, 37, x_dtype, seed=39)
    for M in (1, 3, 8):
        assert vg.plan_variant(fmt, x_dtype, M, 37, K) == VALU
        y_sep, y_sbi = both(vg, case, M, lambda x, w, s, b: vg.verify_gemm(fmt, x, w, s, b))
        assert np.array_equal(y_sep, y_sbi), M
        check(case, M, y_sbi, label="sbi-valu-windows")
