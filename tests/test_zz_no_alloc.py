"""The allocation-free entry point (verify_gemm_argmax_noalloc, static scratch) against the
allocating one it varies (verify_gemm_argmax, and the plain verify call when idx is NULL),
called through the C ABI: the same kernels and plan, so outputs must match bit for bit,
and both must meet the oracle's bar.  Each case makes two calls in a row, the second with
a smaller input; the cases alternate between the paths that use the scratch (K split
across workgroups, the fused argmax, the argmax kernel after the GEMM), so a counter left
non-zero by one call would break the next."""
import numpy as np
import pytest

import oracle
from synthetic import draw_case, workload_case
from synthetic.torch_io import case_tensors

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 2e-3


@pytest.fixture(scope="module")
def vg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import few_row_quantized_verify_amd as m
    m.lib()
    m.force_variant(-1)
    m.force_ksplit(0)
    yield m
    m.force_ksplit(0)


def both(vg, case, M, with_idx, draft=None):
    """(static outputs, allocating outputs) of one call, as numpy arrays."""
    x, w, s, b = case_tensors(case, M)
    dev = x.device
    y0 = torch.full((M, case.N), np.nan, dtype=torch.float32, device=dev)
    y1 = torch.full((M, case.N), -np.nan, dtype=torch.float32, device=dev)
    out0, out1 = [y0], [y1]
    if with_idx:
        i0 = torch.full((M,), -1, dtype=torch.int32, device=dev)
        kw0 = {"idx": i0}
        if draft is not None:
            d = torch.from_numpy(np.asarray(draft[:M], dtype=np.int32)).to(dev)
            a0 = torch.full((1,), -1, dtype=torch.int32, device=dev)
            kw0.update(draft=d, accepted=a0)
        r0 = vg.verify_gemm_argmax_noalloc(case.fmt, x, w, s, b, y0, **kw0)
        r1 = vg.verify_gemm_argmax(case.fmt, x, w, s, b, y=y1,
                                   draft=None if draft is None else kw0["draft"])
        out0, out1 = list(r0), list(r1)
    else:
        vg.verify_gemm_argmax_noalloc(case.fmt, x, w, s, b, y0)
        vg.verify_gemm(case.fmt, x, w, s, b, y=y1)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in out0], [t.cpu().numpy() for t in out1]


def oracle_err(case, M, y):
    ref = oracle.verify(case.fmt, case.x(M), case.x_dtype, case.words, case.scales, case.biases)
    return oracle.normwise_rel_err(y.astype(np.float64), ref)


@pytest.mark.parametrize("name,Ms", [("mlp_down_sign1_k17408_n5120", (8, 3)),   # K split six ways
                                     ("attn_had2_k5120_n6144", (8, 2))])         # K split five ways
def test_split_k_from_static_scratch(vg, name, Ms):
    case = workload_case(name, seed=0)
    assert vg.plan_ksplit(case.fmt, case.x_dtype, Ms[0], case.N, case.K) > 1
    for M in Ms:
        (y0,), (y1,) = both(vg, case, M, with_idx=False)
        assert np.array_equal(y0, y1), f"{name} M={M}: static and allocating calls differ"
        assert oracle_err(case, M, y0) <= TOL


@pytest.mark.parametrize("fmt,K,N,x_dtype,Ms", [("affine2", 5120, 30001, "f16", (8, 5)),   # fused argmax
                                                ("sign1", 512, 256, "f32", (8, 2)),         # VALU + argmax kernel
                                                ("sign1", 17408, 5120, "bf16", (7, 1))])    # split K + argmax kernel
def test_argmax_from_static_scratch(vg, fmt, K, N, x_dtype, Ms):
    case = draw_case(fmt, K, N, x_dtype, seed=90)
    ref_full = oracle.verify(fmt, case.x(8), x_dtype, case.words, case.scales, case.biases)
    ref_idx, _ = oracle.argmax_rows(ref_full)
    draft = ref_idx.copy()
    draft[2] = (draft[2] + 1) % N        # rows 0, 1 agree, row 2 does not
    for M in Ms:
        (y0, i0, a0), (y1, i1, a1) = both(vg, case, M, with_idx=True, draft=draft)
        assert np.array_equal(y0, y1) and np.array_equal(i0, i1) and np.array_equal(a0, a1)
        assert oracle.normwise_rel_err(y0.astype(np.float64), ref_full[:M]) <= TOL
        assert list(i0) == list(ref_idx[:M])
        assert int(a0[0]) == min(M, 2)
        (y0,), (y1,) = both(vg, case, M, with_idx=False)   # and the plain call between
        assert np.array_equal(y0, y1)


def test_static_scratch_limit_is_refused(vg):
    """A call whose split-K partials exceed the static array is refused before anything is
    enqueued (y keeps its contents), and the next call still works."""
    case = draw_case("sign1", 16384, 8192, "bf16", seed=91)
    x, w, s, _ = case_tensors(case, 8)
    y = torch.full((8, case.N), 3.5, dtype=torch.float32, device=x.device)
    vg.force_ksplit(16)
    try:
        with pytest.raises(vg.VerifyGemmError) as e:
            vg.verify_gemm_argmax_noalloc("sign1", x, w, s, None, y)
        assert e.value.status == 5 and "static maximum" in str(e.value)
    finally:
        vg.force_ksplit(0)
    torch.cuda.synchronize()
    assert torch.all(y == 3.5)
    (y0,), (y1,) = both(vg, case, 4, with_idx=False)
    assert np.array_equal(y0, y1)
