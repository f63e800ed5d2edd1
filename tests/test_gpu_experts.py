"""GPU parity of the grouped routed-expert verify, through the C ABI, against the oracle.

Two bars: every routed (row, slot) output meets the same componentwise and normwise
bounds as the plain verify (against the fp64 oracle on the expert it was routed to), and
the grouping is invisible: each slot's output is bit-identical to the output of the same
call with only that row routed ("Ijah" README, "What's new (v0.2)": grouped verify reads
each expert once and gives bit-identical output).
"""
import numpy as np
import pytest

import oracle
from synthetic import Case, EXPERT_WORKLOADS, draw_experts, draw_route
from synthetic.torch_io import case_tensors
from tests.test_gpu_parity import check, sample_cols

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

SENTINEL = 12345.0


@pytest.fixture(scope="module")
def vg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import few_row_quantized_verify_amd as m
    m.lib()
    return m


def run_experts(vg, ec, M, route):
    x, w, s, b = case_tensors(ec, M)
    rt = torch.from_numpy(np.ascontiguousarray(route, dtype=np.int32)).cuda()
    y = torch.full((M, route.shape[1], ec.N), SENTINEL, dtype=torch.float32, device="cuda")
    vg.verify_gemm_experts(ec.fmt, x, rt, w, s, b, y=y)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def check_experts(ec, M, route, y, cols=None, label=""):
    """Each expert's routed slots against the oracle on that expert; unused slots untouched."""
    E = ec.E
    x = ec.x(M)
    used = (route >= 0) & (route < E)
    assert np.all(y[~used] == SENTINEL), f"{label}: an unused slot was written"
    for e in np.unique(route[used]):
        ms, ss = np.nonzero(route == e)
        sub = Case(ec.fmt, ec.K, ec.N, ec.x_dtype, ec.words[e], ec.scales[e],
                   None if ec.biases is None else ec.biases[e], np.ascontiguousarray(x[ms]))
        got = np.zeros((len(ms), ec.N))
        got[:] = y[ms, ss].astype(np.float64)
        check(sub, len(ms), got, cols=cols, label=f"{label} e={e}")


@pytest.mark.parametrize("fmt,x_dtype", [("affine2", "f16"), ("sign1", "bf16"), ("affine1", "bf16"),
                                         ("had2", "f16")])
@pytest.mark.parametrize("M,topk,E", [(1, 8, 16), (3, 2, 5), (4, 4, 8), (5, 3, 12), (8, 8, 16), (8, 1, 3)])
def test_experts_parity(vg, fmt, x_dtype, M, topk, E):
    ec = draw_experts(fmt, 1024, 200, E, x_dtype, seed=M * 10 + topk)
    route = draw_route(M, topk, E, seed=E + M)
    y = run_experts(vg, ec, M, route)
    check_experts(ec, M, route, y, label=f"{fmt} M={M} topk={topk} E={E}")


@pytest.mark.parametrize("M", [1, 4, 5, 8])
def test_grouping_is_bit_identical(vg, M):
    """Each slot's output equals, bit for bit, the output of the same call (same M, topk
    and E) in which only that row is routed."""
    E, topk = 6, 3
    ec = draw_experts("affine2", 2048, 333, E, "f16", seed=70 + M)
    rng = np.random.default_rng(71)
    route = draw_route(M, topk, E, seed=72 + M)
    route[0, 0] = route[M - 1, topk - 1]           # make experts shared between rows
    y = run_experts(vg, ec, M, route)
    for m in range(M):
        alone = np.full_like(route, -1)
        alone[m] = route[m]
        ya = run_experts(vg, ec, M, alone)
        assert np.array_equal(y[m].view(np.uint32), ya[m].view(np.uint32)), f"row {m} differs"
        others = np.arange(M) != m
        assert np.all(ya[others] == SENTINEL)
    # a permutation of the slots moves the outputs with them, unchanged
    perm = rng.permutation(topk)
    yp = run_experts(vg, ec, M, route[:, perm])
    assert np.array_equal(yp.view(np.uint32), y[:, perm].view(np.uint32))


@pytest.mark.parametrize("M", [2, 4, 7, 8])
def test_shared_and_duplicate_experts(vg, M):
    """Every row on the same experts (one job of M rows per expert), and a row routed to
    one expert in several slots (more rows for an expert than a job holds: the expert's
    rows are split over several jobs)."""
    E, topk = 4, 4
    ec = draw_experts("sign1", 1024, 150, E, "f16", seed=80 + M)
    route = np.tile(np.array([[2, 0, 3, 1]], dtype=np.int32), (M, 1))
    check_experts(ec, M, route, run_experts(vg, ec, M, route), label=f"shared M={M}")
    dup = np.full((M, topk), 1, dtype=np.int32)
    dup[:, 3] = 3
    check_experts(ec, M, dup, run_experts(vg, ec, M, dup), label=f"dup M={M}")


def test_unused_and_out_of_range_slots(vg):
    """Slots routed outside 0..E-1 (negative, E, huge) are skipped and left unwritten;
    a routing with no used slot writes nothing."""
    E, M, topk = 5, 6, 4
    ec = draw_experts("affine2", 1024, 77, E, "f16", seed=90)
    route = draw_route(M, topk, E, seed=91)
    route[0, 1] = -1
    route[2, :] = [E, -7, 2 ** 31 - 1, 3]
    route[5, 3] = -(2 ** 31)
    check_experts(ec, M, route, run_experts(vg, ec, M, route), label="unused")
    none = np.full((M, topk), -1, dtype=np.int32)
    assert np.all(run_experts(vg, ec, M, none) == SENTINEL)


def test_consecutive_calls_different_routing(vg):
    """The job table lives in the stream's workspace: calls with different routings, row
    counts and expert counts in a row each read their own."""
    for i, (M, topk, E) in enumerate([(8, 8, 64), (1, 2, 3), (5, 4, 9), (8, 8, 64)]):
        ec = draw_experts("affine2", 1024, 96, E, "f16", seed=100 + i)
        route = draw_route(M, topk, E, seed=110 + i)
        check_experts(ec, M, route, run_experts(vg, ec, M, route), label=f"call{i}")


@pytest.mark.parametrize("M", [1, 8])
def test_moe_workload_sampled(vg, M):
    """The full routed-expert workload (128 experts, 8 per row) on sampled columns."""
    name = "moe_gate_up_affine2_e128_top8_k2048_n1536"
    fmt, K, N, E, topk, x_dtype = EXPERT_WORKLOADS[name]
    ec = draw_experts(fmt, K, N, E, x_dtype, seed=0)
    route = draw_route(M, topk, E, seed=0)
    y = run_experts(vg, ec, M, route)
    cols = sample_cols(N, k=64, seed=M)
    check_experts(ec, M, route, y, cols=cols, label=name)
