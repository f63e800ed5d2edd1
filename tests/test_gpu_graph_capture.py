"""GPU: the verify calls captured in a HIP graph and replayed, against the same calls run
eagerly on the same stream.

A call allocates nothing once its stream's workspace exists (the first call on a stream
sets it up, counters cleared), and every kernel leaves the counters and argmax keys it uses
at zero, so a captured call replays without any memset node.  Each replay runs after eager
work of the test's own (the outputs overwritten with NaN) and a synchronization, and must
give the eager call's bits again: the kernels reduce in a fixed order.
"""
import numpy as np
import pytest

from synthetic import draw_case
from synthetic.torch_io import case_tensors

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def vg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import few_row_quantized_verify_amd as m
    m.lib()  # fails loudly if the library is missing
    m.force_variant(-1)
    m.force_ksplit(0)
    return m


@pytest.mark.parametrize("fmt,K,N,x_dtype,M,argmax,sbi", [
    ("affine2", 2048, 3000, "f16", 8, False, False),    # one K slice, the 8-row variant
    ("sign1", 17408, 5120, "bf16", 4, False, False),    # K split across workgroups: arrival counters
    ("affine2", 2048, 8192, "f16", 6, True, False),     # the fused argmax: keys and arrival counter
    ("sign1", 512, 256, "f32", 8, True, False),         # the VALU kernel, then the argmax kernel
    ("affine2", 2048, 8192, "f16", 6, True, True),      # the same, interleaved scales and biases
    ("affine2", 5120, 4096, "f16", 1, False, True),     # one row: the dot2 kernel, interleaved
])
def test_graph_replays_match_eager(vg, fmt, K, N, x_dtype, M, argmax, sbi):
    case = draw_case(fmt, K, N, x_dtype, seed=80)
    x, w, s, b = case_tensors(case, M)
    if sbi:
        s, b = vg.pack_scale_bias(s, b), None   # packed eagerly, before any capture
    st = torch.cuda.Stream()
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    idx = torch.empty((M,), dtype=torch.int32, device="cuda")

    def call():
        if argmax:
            vg.verify_gemm_argmax(fmt, x, w, s, b, y=y, idx=idx)
        else:
            vg.verify_gemm(fmt, x, w, s, b, y=y)

    torch.cuda.synchronize()
    with torch.cuda.stream(st):
        call()                      # sets up this stream's workspace
    st.synchronize()
    y0 = y.clone()
    idx0 = idx.clone()
    print(f"graph case {fmt} K={K} N={N} {x_dtype} M={M} argmax={argmax} sbi={sbi} "
          f"ksplit={vg.plan_ksplit(fmt, x_dtype, M, N, K)}", flush=True)

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=st):
        call()
    torch.cuda.synchronize()
    for r in range(3):
        y.fill_(float("nan"))
        idx.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y0), f"replay {r}: logits differ from the eager call"
        if argmax:
            assert torch.equal(idx, idx0), f"replay {r}: argmax differs from the eager call"
            assert np.array_equal(idx.cpu().numpy(), np.argmax(y.cpu().numpy(), axis=1))
    del g
