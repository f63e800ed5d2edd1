"""GPU: the verify GEMM with the argmax of every row in one call (verify_gemm_argmax),
through the C ABI, against the plain GEMM, the argmax kernel and the fp64 oracle.

The output head's verify is checked by its argmax ("dflash-mlx-bonsai2" README, "Verify it
yourself"); the rule is the largest value, the lowest column on ties, NaN never winning.
"""
import json
import os

import numpy as np
import pytest

import oracle
from synthetic import draw_case, workload_case
from synthetic.torch_io import case_tensors

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.fixture(scope="module")
def vg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import few_row_quantized_verify_amd as m
    m.lib()  # fails loudly if the library is missing
    m.force_variant(-1)
    m.force_ksplit(0)
    return m


def plain(vg, case, M):
    x, w, s, b = case_tensors(case, M)
    y = vg.verify_gemm(case.fmt, x, w, s, b)
    return y, vg.verify_argmax_rows(y)


def fused(vg, case, M, draft=None):
    x, w, s, b = case_tensors(case, M)
    d = None if draft is None else torch.from_numpy(np.asarray(draft, dtype=np.int32)).cuda()
    return vg.verify_gemm_argmax(case.fmt, x, w, s, b, draft=d)


class same_gemm:
    """Pins plain and argmax calls to the variant the argmax call runs, so the two run the same
    GEMM: where the dispatch gives a plain one-row call the dot2 kernel, the argmax call runs
    mode Q (its epilogue fuses the argmax); elsewhere both run the plain call's variant."""

    def __init__(self, vg, case, M):
        v = vg.plan_variant(case.fmt, case.x_dtype, M, case.N, case.K)
        self.vg, self.var = vg, 0 if vg.variant_name(v) == "vg_gemv" else v   # 0: vg_mfma_q

    def __enter__(self):
        self.vg.force_variant(self.var)

    def __exit__(self, *exc):
        self.vg.force_variant(-1)


def test_head_fused_matches_oracle_and_plain_path(vg):
    """Output-head shape (one K slice: the fused epilogue runs): y bit-identical to the plain
    call, idx equal to the oracle's argmax stored with the workload, at every ragged M."""
    with open(os.path.join(GOLDEN, "head_affine2_k5120_n151936_argmax.json")) as f:
        gold = json.load(f)
    case = workload_case(gold["workload"], seed=gold["seed"])
    assert vg.plan_ksplit("affine2", "f16", 8, case.N, case.K) == 1
    for M in (8, 5, 6, 7, 1):
        with same_gemm(vg, case, M):
            y, idx = fused(vg, case, M)
            y0, idx0 = plain(vg, case, M)
        torch.cuda.synchronize()
        assert torch.equal(y, y0), f"M={M}: fused call changed the logits"
        got = idx.cpu().numpy()
        print(f"head M={M} idx={list(got)}", flush=True)
        assert list(got) == gold["argmax"][:M]
        assert np.array_equal(got, idx0.cpu().numpy())


def test_head_fused_accept(vg):
    with open(os.path.join(GOLDEN, "head_affine2_k5120_n151936_argmax.json")) as f:
        gold = json.load(f)
    case = workload_case(gold["workload"], seed=gold["seed"])
    M = 7
    for k in (0, 3, M):
        draft = np.array(gold["argmax"][:M], dtype=np.int32)
        if k < M:
            draft[k] = (draft[k] + 11) % case.N
        y, idx, acc = fused(vg, case, M, draft)
        assert list(idx.cpu().numpy()) == gold["argmax"][:M]
        assert int(acc.cpu().numpy()[0]) == k


@pytest.mark.parametrize("fmt,K,N,x_dtype", [
    ("affine2", 2048, 5000, "f16"),
    ("sign1", 2048, 4099, "bf16"),
    ("affine1", 1024, 3001, "bf16"),
    ("had2", 1024, 2050, "f16"),
    ("sign1", 512, 256, "f32"),          # the VALU kernel: the argmax kernel runs after it
    ("sign1", 17408, 5120, "bf16"),      # K split across workgroups: likewise
])
def test_fused_equals_separate_argmax(vg, fmt, K, N, x_dtype):
    case = draw_case(fmt, K, N, x_dtype, seed=60)
    for M in (1, 4, 8):
        with same_gemm(vg, case, M):
            y, idx = fused(vg, case, M)
            y0, idx0 = plain(vg, case, M)
        torch.cuda.synchronize()
        assert torch.equal(y, y0)
        got = idx.cpu().numpy()
        assert np.array_equal(got, idx0.cpu().numpy())
        assert np.array_equal(got, np.argmax(y.cpu().numpy(), axis=1))


def test_fused_ties_pick_the_lowest_column(vg):
    """All-zero scales make every logit a (signed) zero: every column ties, across every
    workgroup, and the lowest column (0) must win; -0 ties with +0."""
    case = draw_case("sign1", 1024, 3000, "bf16", seed=61)
    case.scales = np.zeros_like(case.scales)
    for M in (1, 8):
        y, idx = fused(vg, case, M)
        assert torch.all(y == 0)
        assert list(idx.cpu().numpy()) == [0] * M


def test_fused_planted_winner_in_last_workgroup(vg):
    """A single column made the winner by its weights, in the last row group, and the same
    value planted twice in different workgroups (the lower column wins)."""
    case = draw_case("affine2", 1024, 4096, "f16", seed=62)
    for col in (4095, 100):
        case.scales[col] = np.uint16(0)          # scale 0: w = b exactly
        case.biases[col] = np.uint16(0x5800)     # b = 128: y = 128 * sum(x)
    x = oracle.activations(case.x(8), "f16")
    want = np.where(x.sum(axis=1) > 0, 100, None)
    y, idx = fused(vg, case, 8)
    got = idx.cpu().numpy()
    y_np = y.cpu().numpy()
    assert np.array_equal(got, np.argmax(y_np, axis=1))
    for m in range(8):
        if want[m] is not None and y_np[m, 100] == y_np[m].max():
            assert got[m] == 100   # ties with column 4095: the lower column


def test_fused_consecutive_calls_reset_state(vg):
    """Each call overwrites the key slots of its own workgroups and rows, and the pick reads
    only those: a large M, then a smaller one on other inputs (the higher rows' slots keep
    the earlier call's keys), then a shape with far fewer workgroups (the later workgroups'
    slots keep theirs), then the first again, on one stream."""
    a = draw_case("affine2", 2048, 6000, "f16", seed=63)
    b = draw_case("affine2", 2048, 6000, "f16", seed=64)
    c = draw_case("affine2", 2048, 300, "f16", seed=65)   # 19 tiles: 19 workgroups
    for case, M in ((a, 8), (b, 3), (c, 8), (a, 8), (b, 8), (c, 2)):
        y, idx = fused(vg, case, M)
        assert np.array_equal(idx.cpu().numpy(), np.argmax(y.cpu().numpy(), axis=1)), (case.N, M)


@pytest.mark.parametrize("K,N,direct", [(2048, 300, 0), (5120, 12000, 1)])
def test_fused_nan_rows_give_column_zero(vg, K, N, direct):
    """A drafted row of NaN activations makes every logit of that row NaN: no workgroup has a
    key for it and its idx is 0, while the other rows keep their own argmax; the accepted
    count stops at the first row whose argmax differs from the draft.  Both finishes: the
    barrier one and the direct one, whose waves fold the keys as they store."""
    case = draw_case("affine2", K, N, "f16", seed=66)
    M = 6
    assert vg.plan_direct("affine2", "f16", M, N, K) == direct
    x, w, s, b = case_tensors(case, M)
    x[2] = float("nan")
    y, idx = vg.verify_gemm_argmax(case.fmt, x, w, s, b)
    torch.cuda.synchronize()
    y_np = y.cpu().numpy()
    assert np.all(np.isnan(y_np[2])) and not np.any(np.isnan(np.delete(y_np, 2, axis=0)))
    want = np.argmax(np.where(np.isnan(y_np), -np.inf, y_np), axis=1)
    want[2] = 0
    assert np.array_equal(idx.cpu().numpy(), want)
    draft = torch.from_numpy(want.astype(np.int32)).cuda()
    draft[3] += 1
    _, idx2, acc = vg.verify_gemm_argmax(case.fmt, x, w, s, b, draft=draft)
    torch.cuda.synchronize()
    assert np.array_equal(idx2.cpu().numpy(), want) and int(acc[0]) == 3


def test_one_row_argmax_call_keeps_the_fused_kernel(vg):
    """A plain one-row call of an affine shape runs vg_gemv; the same call with the argmax runs
    mode Q, whose epilogue fuses it.  The two logits agree to the verify bar, and idx is the
    argmax of the call's own logits."""
    for fmt, x_dtype in (("affine2", "f16"), ("affine1", "bf16")):
        case = draw_case(fmt, 2048, 5000, x_dtype, seed=61)
        assert vg.variant_name(vg.plan_variant(fmt, x_dtype, 1, case.N, case.K)) == "vg_gemv"
        y, idx = fused(vg, case, 1)
        y0, _ = plain(vg, case, 1)
        torch.cuda.synchronize()
        a, b = y.cpu().numpy().astype(np.float64), y0.cpu().numpy().astype(np.float64)
        assert np.max(np.abs(a - b)) <= 2e-3 * np.max(np.abs(b)), fmt
        assert int(idx.cpu()[0]) == int(np.argmax(y.cpu().numpy()[0])), fmt
