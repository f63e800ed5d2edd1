"""GPU: the two ways an MFMA workgroup finishes its output tiles give the same bits.

A plain verify whose K fits one LDS staging window, in one K slice, with at least as many
units for every wave as it loads ahead, stores each 16-row tile from the wave that completes
it: a tile that waves share is added up, in wave order, by the last of them to arrive (a
counter in LDS), and no barrier follows the main loop.  Every other call, and every call
under vg_force_barrier_tail, meets at a workgroup barrier and adds the shared tiles after
it.  The two are the same sums in the same order, so the outputs must be bit-identical.
The shapes make every kind of tile occur: K = 1024 (one K-step, so every unit is a whole
tile held by one wave), K = 2048 (tiles held by one wave beside shared ones), K = 5120
(every tile shared by two or three waves), ragged last tiles (N not a multiple of 16), in
both MFMA row-block modes, every format, both layouts of the affine scales and biases.
Outputs start as NaN, so an element neither finish writes fails the comparison, and one
shape per format is also held to the fp64 oracle's bounds.
"""
import numpy as np
import pytest

from synthetic import draw_case
from synthetic.torch_io import case_tensors
from tests.test_gpu_parity import check, reference

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

Q, H = 0, 1
SHAPES = [(1024, 40000), (2048, 40003), (5120, 17411), (3072, 9000)]
ORACLE_SHAPE = (2048, 40003)


@pytest.fixture(scope="module")
def vg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import few_row_quantized_verify_amd as m
    m.lib()  # fails loudly if the library is missing
    m.force_variant(-1)
    m.force_ksplit(0)
    m.force_barrier_tail(False)
    yield m
    m.force_variant(-1)
    m.force_ksplit(0)
    m.force_barrier_tail(False)


def run(vg, fmt, x, w, s, b, M, N):
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    vg.verify_gemm(fmt, x, w, s, b, y=y)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("fmt", ["sign1", "affine2", "had2", "affine1"])
@pytest.mark.parametrize("x_dtype", ["f16", "bf16"])
def test_direct_and_barrier_tails_agree(vg, fmt, x_dtype):
    direct_runs = {Q: 0, H: 0}
    try:
        for K, N in SHAPES:
            case = draw_case(fmt, K, N, x_dtype, seed=K + N)
            ref = reference(case, 8) if (K, N) == ORACLE_SHAPE and x_dtype == "f16" else None
            for v in (Q, H):
                vg.force_variant(v)
                for M in range(1, 9):
                    if vg.plan_variant(fmt, x_dtype, M, N, K) != v:
                        continue
                    direct = vg.plan_direct(fmt, x_dtype, M, N, K)
                    assert direct in (0, 1), (K, N, v, M)
                    direct_runs[v] += direct
                    x, w, s, b = case_tensors(case, M)
                    layouts = [(s, b)] + ([(vg.pack_scale_bias(s, b), None)] if b is not None else [])
                    for s_, b_ in layouts:
                        y_dir = run(vg, fmt, x, w, s_, b_, M, N)
                        vg.force_barrier_tail(True)
                        try:
                            assert vg.plan_direct(fmt, x_dtype, M, N, K) == 0
                            y_bar = run(vg, fmt, x, w, s_, b_, M, N)
                        finally:
                            vg.force_barrier_tail(False)
                        assert not torch.isnan(y_bar).any(), (K, N, v, M)
                        assert torch.equal(y_dir, y_bar), (fmt, x_dtype, K, N, vg.variant_name(v), M, direct)
                    if ref is not None:
                        check(case, M, y_dir.cpu().numpy().astype(np.float64), ref=ref,
                              label=f"direct[{vg.variant_name(v)}]")
    finally:
        vg.force_variant(-1)
    # the shapes must reach the direct finish in both row-block modes
    assert direct_runs[Q] > 0 and direct_runs[H] > 0, direct_runs


def test_split_k_and_long_k_take_the_barrier(vg):
    """The plan's own bounds: a K split, or a K longer than one window, never finishes
    directly (their tiles are summed across slices or windows after the barrier)."""
    try:
        vg.force_ksplit(2)
        assert vg.plan_direct("affine2", "f16", 8, 17408, 5120) == 0
        vg.force_ksplit(1)
        assert vg.plan_direct("affine2", "f16", 8, 300, 16384) == 0
    finally:
        vg.force_ksplit(0)
    assert vg.plan_direct("affine2", "f32", 4, 17408, 5120) == 0    # the VALU kernel
    assert vg.plan_direct("affine2", "f16", 8, 17408, 5120) == 1    # the 2-bit MLP up-projection


def test_one_row_affine1_takes_mode_q_when_it_finishes_directly(vg):
    """The dispatch at one row of the 1-bit affine format: mode Q where its tiles finish
    without the barrier, the dot2 kernel elsewhere (as for the 2-bit format everywhere)."""
    Qname, G = "vg_mfma_q", "vg_gemv"
    for K, N in ((5120, 17408), (2048, 5000), (1024, 333)):
        direct = vg.plan_direct("affine1", "bf16", 1, N, K)
        vg.force_variant(Q)
        try:
            q_direct = vg.plan_direct("affine1", "bf16", 1, N, K)
        finally:
            vg.force_variant(-1)
        assert vg.variant_name(vg.plan_variant("affine1", "bf16", 1, N, K)) == (Qname if q_direct else G), (K, N)
        assert direct == q_direct, (K, N)
        assert vg.variant_name(vg.plan_variant("affine2", "f16", 1, N, K)) == G, (K, N)
    vg.force_variant(Q)
    try:
        assert vg.plan_direct("affine1", "bf16", 1, 17408, 5120) == 1
        assert vg.plan_direct("affine1", "bf16", 1, 333, 1024) == 0
    finally:
        vg.force_variant(-1)


# Six-wave staging: a mode-Q launch whose staging window holds more than 384 and at most 512
# chunks (32 K of one row each, M * 32 per 1024-K step) stages on the first six waves only.
# The cases below reach it with the barrier finish: with the fused argmax (K = 5120 at three
# rows, 480 chunks; K = 4096 at four rows, 512; N large enough that K stays in one slice,
# which the fused argmax needs) and with K split over two slices (K = 8192, a 4-step window
# per slice, 512 chunks at four rows; 384 at three rows, which keeps eight waves).  Every output is held to the oracle's
# bounds; the argmax to the argmax of the call's own logits and of the oracle's.

@pytest.mark.parametrize("fmt,K,N,x_dtype,M", [("affine2", 5120, 12000, "f16", 3), ("sign1", 5120, 12001, "bf16", 3),
                                               ("affine1", 4096, 12003, "bf16", 4), ("affine2", 4096, 16384, "f16", 4)])
def test_six_wave_staging_with_the_fused_argmax(vg, fmt, K, N, x_dtype, M):
    case = draw_case(fmt, K, N, x_dtype, seed=K + N + M)
    assert vg.plan_variant(fmt, x_dtype, M, N, K) == Q
    assert vg.plan_ksplit(fmt, x_dtype, M, N, K) == 1
    x, w, s, b = case_tensors(case, M)
    y, idx = vg.verify_gemm_argmax(fmt, x, w, s, b)
    torch.cuda.synchronize()
    yn = y.cpu().numpy().astype(np.float64)
    ref = reference(case, M)
    check(case, M, yn, ref=ref, label="six-wave+argmax")
    assert idx.cpu().tolist() == list(np.argmax(y.cpu().numpy(), axis=1))
    # the oracle's argmax, wherever its top two are apart by more than the verify bar
    y_ref = ref[0]
    for m in range(M):
        top2 = np.sort(y_ref[m])[-2:]
        if top2[1] - top2[0] > 4e-3 * np.max(np.abs(y_ref[m])):
            assert int(idx[m]) == int(np.argmax(y_ref[m])), m


@pytest.mark.parametrize("fmt,x_dtype", [("affine2", "f16"), ("sign1", "bf16"), ("affine1", "bf16")])
def test_six_wave_staging_with_k_split(vg, fmt, x_dtype):
    K, N = 8192, 300
    case = draw_case(fmt, K, N, x_dtype, seed=91)
    try:
        vg.force_ksplit(2)
        for M in (3, 4):
            assert vg.plan_variant(fmt, x_dtype, M, N, K) == Q
            assert vg.plan_ksplit(fmt, x_dtype, M, N, K) == 2
            x, w, s, b = case_tensors(case, M)
            y = run(vg, fmt, x, w, s, b, M, N)
            check(case, M, y.cpu().numpy().astype(np.float64), label=f"six-wave+ksplit M={M}")
    finally:
        vg.force_ksplit(0)


@pytest.mark.parametrize("fmt,K,N,x_dtype", [("affine2", 5120, 12000, "f16"), ("sign1", 5120, 13001, "bf16"),
                                             ("affine1", 2048, 40003, "bf16"), ("had2", 1024, 40000, "f16")])
def test_argmax_direct_and_barrier_finishes_agree(vg, fmt, K, N, x_dtype):
    """The fused argmax on the direct finish (each wave folds the keys of the tiles it stores,
    the workgroup's last wave stores them) against the barrier finish: logits, idx and the
    accepted count bit for bit, with a draft that agrees on a prefix."""
    case = draw_case(fmt, K, N, x_dtype, seed=K + N + 5)
    ran = 0
    for M in range(1, 9):
        x, w, s, b = case_tensors(case, M)
        direct = vg.plan_direct(fmt, x_dtype, M, N, K)
        ran += direct
        outs = []
        for bar in (False, True):
            vg.force_barrier_tail(bar)
            try:
                y, idx = vg.verify_gemm_argmax(fmt, x, w, s, b)
                torch.cuda.synchronize()
                draft = idx.clone()
                if M > 1:
                    draft[M // 2] += 1   # agrees on the first M // 2 rows only
                _, idx2, acc = vg.verify_gemm_argmax(fmt, x, w, s, b, draft=draft)
                torch.cuda.synchronize()
            finally:
                vg.force_barrier_tail(False)
            outs.append((y.clone(), idx.clone(), idx2.clone(), int(acc[0])))
        (y0, i0, j0, a0), (y1, i1, j1, a1) = outs
        assert torch.equal(y0, y1) and torch.equal(i0, i1) and torch.equal(j0, i0) and a0 == a1, (M, direct)
        assert a0 == (M if M == 1 else M // 2), (M, a0)
        assert i0.cpu().tolist() == list(np.argmax(y0.cpu().numpy(), axis=1)), M
    assert ran > 0   # the shapes reach the direct finish
