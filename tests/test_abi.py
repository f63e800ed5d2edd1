"""CPU tests of the C ABI: the library loads, exports what the header declares, and
rejects every invalid argument with its status before touching a device."""
import ctypes
import os
import re

import pytest

import few_row_quantized_verify_amd as vgm
from few_row_quantized_verify_amd import binding as B

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "verify_gemm.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?(?:vg_status|int|const char\*|char\*)\s*\*?\s*(\w+)\s*\(", src, flags=re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for fn in ("verify_gemm_sign1", "verify_gemm_affine2", "verify_gemm_had2", "hadamard_rotate",
               "verify_argmax_rows", "vg_last_error", "vg_plan_variant", "vg_variant_name",
               "vg_force_variant", "vg_variant_count", "vg_debug_unpack_sign1", "vg_debug_unpack_affine2",
               "vg_plan_ksplit", "vg_force_ksplit", "verify_accept_greedy", "verify_gemm_affine1",
               "verify_gemm_had2_signed", "hadamard_rotate_signed", "verify_gemm_experts",
               "verify_gemm_argmax", "vg_debug_unpack", "vg_release_stream_workspace", "vg_stream_read_config",
               "vg_pack_scale_bias", "vg_plan_direct", "vg_force_barrier_tail"):
        assert fn in names, fn


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(B.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_binding_signatures_cover_header():
    assert set(declared_functions()) == set(B._SIGS)


ALIGNED = 1 << 20   # a fake, 16-byte aligned address: never dereferenced on the error paths
MISALIGNED = ALIGNED + 4


def _err():
    return B.lib().vg_last_error().decode()


@pytest.mark.parametrize("M", [0, -1, 9, 100])
def test_bad_row_count(M):
    st = B.lib().verify_gemm_sign1(ALIGNED, B.VG_F16, M, 512, ALIGNED, ALIGNED, 256, ALIGNED, None)
    assert st == B.VG_ERR_SHAPE and "M=" in _err()


def test_bad_n_and_k():
    L = B.lib()
    assert L.verify_gemm_sign1(ALIGNED, B.VG_F16, 1, 512, ALIGNED, ALIGNED, 0, ALIGNED, None) == B.VG_ERR_SHAPE
    assert L.verify_gemm_sign1(ALIGNED, B.VG_F16, 1, 500, ALIGNED, ALIGNED, 8, ALIGNED, None) == B.VG_ERR_SHAPE
    assert L.verify_gemm_sign1(ALIGNED, B.VG_F16, 1, 64, ALIGNED, ALIGNED, 8, ALIGNED, None) == B.VG_ERR_SHAPE
    assert L.verify_gemm_affine2(ALIGNED, B.VG_F16, 1, 96, ALIGNED, ALIGNED, ALIGNED, 8, ALIGNED, None) == B.VG_ERR_SHAPE
    assert L.verify_gemm_had2(ALIGNED, B.VG_F16, 1, 192, ALIGNED, ALIGNED, ALIGNED, 8, 128, ALIGNED, None) == B.VG_ERR_SHAPE
    assert L.hadamard_rotate(ALIGNED, B.VG_F16, 1, 200, 128, ALIGNED, None) == B.VG_ERR_SHAPE
    assert L.verify_argmax_rows(ALIGNED, 1, 0, ALIGNED, None) == B.VG_ERR_SHAPE
    assert L.verify_argmax_rows(ALIGNED, 9, 10, ALIGNED, None) == B.VG_ERR_SHAPE


def test_bad_dtype():
    st = B.lib().verify_gemm_affine2(ALIGNED, 7, 1, 256, ALIGNED, ALIGNED, ALIGNED, 8, ALIGNED, None)
    assert st == B.VG_ERR_DTYPE and "dtype" in _err()


@pytest.mark.parametrize("which", [0, 1, 2, 4])
def test_null_pointers(which):
    ptrs = [ALIGNED] * 5
    ptrs[which] = None
    x, w, s, b, y = ptrs
    st = B.lib().verify_gemm_affine2(x, B.VG_F16, 2, 256, w, s, b, 8, y, None)
    assert st == B.VG_ERR_ARG and "null" in _err()


def test_null_biases_select_the_interleaved_layout():
    """NULL biases of an affine format mean interleaved (scale, bias) pairs in scales, not an
    error; misaligned biases are still refused.  (Bad row counts are checked first, so these
    calls stop before touching a device.)"""
    L = B.lib()
    assert L.verify_gemm_affine2(ALIGNED, B.VG_F16, 9, 256, ALIGNED, ALIGNED, None, 8, ALIGNED, None) == B.VG_ERR_SHAPE
    assert L.verify_gemm_affine2(ALIGNED, B.VG_F16, 2, 256, ALIGNED, ALIGNED, MISALIGNED, 8, ALIGNED,
                                 None) == B.VG_ERR_ALIGN
    assert L.verify_gemm_affine1(ALIGNED, B.VG_F16, 2, 256, ALIGNED, ALIGNED, MISALIGNED, 8, ALIGNED,
                                 None) == B.VG_ERR_ALIGN
    assert L.verify_gemm_had2(ALIGNED, B.VG_F16, 2, 256, ALIGNED, ALIGNED, MISALIGNED, 8, 128, ALIGNED,
                              None) == B.VG_ERR_ALIGN


def test_pack_scale_bias_validation():
    L = B.lib()
    assert L.vg_pack_scale_bias(ALIGNED, ALIGNED * 2, -1, ALIGNED * 4, None) == B.VG_ERR_SHAPE
    assert L.vg_pack_scale_bias(None, ALIGNED * 2, 8, ALIGNED * 4, None) == B.VG_ERR_ARG
    assert L.vg_pack_scale_bias(ALIGNED, None, 8, ALIGNED * 4, None) == B.VG_ERR_ARG
    assert L.vg_pack_scale_bias(ALIGNED, ALIGNED * 2, 8, None, None) == B.VG_ERR_ARG
    assert L.vg_pack_scale_bias(MISALIGNED, ALIGNED * 2, 8, ALIGNED * 4, None) == B.VG_ERR_ALIGN
    assert L.vg_pack_scale_bias(ALIGNED, ALIGNED * 2, 8, ALIGNED * 4 + 8, None) == B.VG_ERR_ALIGN
    # out [2 * count] uint16 overlapping either input (every call here fails validation:
    # the fake addresses are never dereferenced)
    assert L.vg_pack_scale_bias(ALIGNED, ALIGNED * 2, 8, ALIGNED - 16, None) == B.VG_ERR_ARG
    assert "overlap" in _err()
    assert L.vg_pack_scale_bias(ALIGNED * 4, ALIGNED * 2, 8, ALIGNED * 2 - 16, None) == B.VG_ERR_ARG


@pytest.mark.parametrize("which", range(4))
def test_misaligned_pointers(which):
    ptrs = [ALIGNED] * 4
    ptrs[which] = MISALIGNED
    x, w, s, y = ptrs
    st = B.lib().verify_gemm_sign1(x, B.VG_BF16, 2, 512, w, s, 8, y, None)
    assert st == B.VG_ERR_ALIGN and "aligned" in _err()


@pytest.mark.parametrize("block", [0, 32, 512, 127])
def test_unsupported_hadamard_block_is_refused(block):
    L = B.lib()
    st = L.verify_gemm_had2(ALIGNED, B.VG_F16, 1, 256, ALIGNED, ALIGNED, ALIGNED, 8, block, ALIGNED, None)
    assert st == B.VG_ERR_UNSUPPORTED and "Hadamard block" in _err()
    assert L.hadamard_rotate(ALIGNED, B.VG_F16, 1, 256, block, ALIGNED, None) == B.VG_ERR_UNSUPPORTED


def test_debug_unpack_validation():
    L = B.lib()
    assert L.vg_debug_unpack_sign1(ALIGNED, 4, 48, ALIGNED, None) == B.VG_ERR_SHAPE
    assert L.vg_debug_unpack_affine2(None, 4, 64, ALIGNED, None) == B.VG_ERR_ARG
    assert L.vg_debug_unpack_affine2(ALIGNED, 0, 64, ALIGNED, None) == B.VG_ERR_SHAPE


def test_variants_and_forcing():
    names = [vgm.variant_name(i) for i in range(vgm.variant_count())]
    assert names == ["vg_mfma_q", "vg_mfma_h", "vg_valu", "vg_gemv"]
    assert vgm.variant_name(99) == ""
    with pytest.raises(vgm.VerifyGemmError) as e:
        vgm.force_variant(99)
    assert e.value.status == B.VG_ERR_ARG
    vgm.force_variant(-1)


def test_plan_rejects_invalid_shapes():
    assert vgm.plan_variant("sign1", "f16", 0, 16, 512) == -1
    assert vgm.plan_variant("sign1", "f16", 9, 16, 512) == -1
    assert vgm.plan_variant("affine2", "f16", 1, 16, 100) == -1


def test_python_binding_rejects_unknown_dtype():
    torch = pytest.importorskip("torch")
    x = torch.zeros((1, 128), dtype=torch.int32)
    with pytest.raises(vgm.VerifyGemmError) as e:
        vgm.verify_gemm_sign1(x, x, x)
    assert e.value.status == B.VG_ERR_DTYPE


def test_force_ksplit_validation():
    with pytest.raises(vgm.VerifyGemmError) as e:
        vgm.force_ksplit(-1)
    assert e.value.status == B.VG_ERR_ARG
    with pytest.raises(vgm.VerifyGemmError):
        vgm.force_ksplit(65)
    vgm.force_ksplit(0)
    assert vgm.plan_ksplit("sign1", "f16", 0, 16, 1024) == -1


def test_force_barrier_tail_validation():
    L = B.lib()
    assert L.vg_force_barrier_tail(2) == B.VG_ERR_ARG
    assert L.vg_force_barrier_tail(-1) == B.VG_ERR_ARG
    vgm.force_barrier_tail(True)
    vgm.force_barrier_tail(False)
    assert vgm.plan_direct("sign1", "f16", 0, 16, 1024) == -1   # M = 0: no call takes it
    assert vgm.plan_direct("affine2", "f16", 1, 16, 100) == -1  # K not a multiple of the group


def test_accept_greedy_validation():
    L = B.lib()
    assert L.verify_accept_greedy(ALIGNED, 2, 100, None, ALIGNED, ALIGNED, None) == B.VG_ERR_ARG
    assert L.verify_accept_greedy(ALIGNED, 2, 100, ALIGNED, ALIGNED, None, None) == B.VG_ERR_ARG
    assert L.verify_accept_greedy(ALIGNED, 9, 100, ALIGNED, ALIGNED, ALIGNED, None) == B.VG_ERR_SHAPE
    assert L.verify_accept_greedy(ALIGNED + 2, 2, 100, ALIGNED, ALIGNED, ALIGNED, None) == B.VG_ERR_ALIGN


def test_gemm_argmax_validation():
    """Every argument check of the fused GEMM + argmax call runs on the host, before any
    device work."""
    L = B.lib()
    A, F16 = ALIGNED, B.VG_F16

    def call(fmt=1, x=A, xt=F16, M=2, K=1024, w=A, s=A, b=A, N=64, y=A, idx=A, d=None, acc=None):
        return L.verify_gemm_argmax(fmt, x, xt, M, K, w, s, b, N, y, idx, d, acc, None)

    assert call(fmt=7) == B.VG_ERR_ARG
    assert call(idx=None) == B.VG_ERR_ARG
    assert call(idx=A + 2) == B.VG_ERR_ALIGN
    assert call(d=A) == B.VG_ERR_ARG
    assert call(acc=A) == B.VG_ERR_ARG
    assert call(M=9) == B.VG_ERR_SHAPE
    assert call(M=0) == B.VG_ERR_SHAPE
    assert call(fmt=0, K=1088) == B.VG_ERR_SHAPE      # 1-bit groups of 128
    assert call(fmt=2, K=1088) == B.VG_ERR_SHAPE      # rotated blocks of 128
    assert call(b=A + 4) == B.VG_ERR_ALIGN
    # null biases select the interleaved pairs: validation goes on to y
    assert call(b=None, y=None) == B.VG_ERR_ARG and "y is null" in _err()
    assert call(xt=5) == B.VG_ERR_DTYPE
    assert call(y=None) == B.VG_ERR_ARG


def test_hadamard_block_must_divide_k_and_signs_aligned():
    L = B.lib()
    assert L.verify_gemm_had2(ALIGNED, B.VG_F16, 1, 384, ALIGNED, ALIGNED, ALIGNED, 8, 256, ALIGNED, None) == B.VG_ERR_SHAPE
    assert L.hadamard_rotate(ALIGNED, B.VG_F16, 1, 192, 128, ALIGNED, None) == B.VG_ERR_SHAPE
    assert L.verify_gemm_had2_signed(ALIGNED, B.VG_F16, 1, 256, ALIGNED, ALIGNED, ALIGNED, 8, 64, ALIGNED + 2,
                                     ALIGNED, None) == B.VG_ERR_ALIGN
    assert L.hadamard_rotate_signed(ALIGNED, B.VG_F16, 1, 256, 64, ALIGNED + 1, ALIGNED, None) == B.VG_ERR_ALIGN


def test_experts_validation():
    L = B.lib()
    A = ALIGNED

    def call(fmt=B.FMT_AFFINE2, x=A, xt=B.VG_F16, M=2, K=2048, E=8, topk=4, route=A, w=A, s=A, b=A, N=64, y=A):
        return L.verify_gemm_experts(fmt, x, xt, M, K, E, topk, route, w, s, b, N, y, None)

    assert call(fmt=4) == B.VG_ERR_ARG and "format" in _err()
    assert call(fmt=-1) == B.VG_ERR_ARG
    assert call(M=0) == B.VG_ERR_SHAPE
    assert call(M=9) == B.VG_ERR_SHAPE
    assert call(E=0) == B.VG_ERR_SHAPE
    assert call(topk=0) == B.VG_ERR_SHAPE
    assert call(topk=9) == B.VG_ERR_SHAPE
    assert call(N=0) == B.VG_ERR_SHAPE
    assert call(xt=B.VG_F32) == B.VG_ERR_UNSUPPORTED and "fp16 or bf16" in _err()
    assert call(xt=7) == B.VG_ERR_DTYPE
    assert call(K=1536) == B.VG_ERR_UNSUPPORTED and "1024" in _err()
    assert call(route=None) == B.VG_ERR_ARG and "route" in _err()
    assert call(route=A + 2) == B.VG_ERR_ALIGN
    assert call(w=None) == B.VG_ERR_ARG
    assert call(s=A + 4) == B.VG_ERR_ALIGN
    assert call(b=A + 4) == B.VG_ERR_ALIGN and "biases" in _err()
    # null biases select the interleaved pairs [E, N, K/G, 2]: validation goes on to y
    for fmt in (B.FMT_AFFINE2, B.FMT_HAD2, B.FMT_AFFINE1):
        assert call(fmt=fmt, b=None, y=None) == B.VG_ERR_ARG and "y is null" in _err()
    assert call(y=A + 8) == B.VG_ERR_ALIGN
    assert call(x=None) == B.VG_ERR_ARG


def test_stream_read_validation():
    L = B.lib()
    assert L.vg_stream_read(None, 1024, ALIGNED, None) == B.VG_ERR_ARG
    assert L.vg_stream_read(ALIGNED + 4, 1024, ALIGNED, None) == B.VG_ERR_ALIGN
    assert L.vg_stream_read(ALIGNED, 0, ALIGNED, None) == B.VG_ERR_SHAPE
    assert L.vg_stream_read(ALIGNED, 1000, ALIGNED, None) == B.VG_ERR_SHAPE
    assert L.vg_stream_read(ALIGNED, 1024, None, None) == B.VG_ERR_ARG
    assert L.vg_stream_read(ALIGNED, 1024, ALIGNED + 2, None) == B.VG_ERR_ALIGN
    for lif, wgs in ((3, 8), (0, 8), (32, 8), (4, 0), (4, 33)):
        assert L.vg_stream_read_config(ALIGNED, 1024, ALIGNED, lif, wgs, None) == B.VG_ERR_ARG


# ----------------------------------------------------------------------------- binding checks
# The C ABI sees raw pointers and cannot check what they point to, so the Python binding
# checks shape, dtype, contiguity and device before any call into the library.  Each case
# below is caught on the host; CPU tensors of the right shape reach the device check last.
def _affine2_tensors(torch, M=2, K=1024, N=48, xdt=None):
    x = torch.zeros((M, K), dtype=xdt or torch.float16)
    w = torch.zeros((N, K // 16), dtype=torch.int32)
    s = torch.zeros((N, K // 64), dtype=torch.float16)
    b = torch.zeros((N, K // 64), dtype=torch.float16)
    return x, w, s, b


def _raises(status, fn, *a, **kw):
    with pytest.raises(vgm.VerifyGemmError) as e:
        fn(*a, **kw)
    assert e.value.status == status, str(e.value)
    return str(e.value)


def test_binding_checks_weight_shapes_against_the_format():
    torch = pytest.importorskip("torch")
    x, w, s, b = _affine2_tensors(torch)
    # 1-bit words handed to the 2-bit call (half the words a row needs), and the reverse
    w1 = torch.zeros((48, 1024 // 32), dtype=torch.int32)
    assert "w has shape" in _raises(B.VG_ERR_SHAPE, vgm.verify_gemm_affine2, x, w1, s, b)
    s1 = torch.zeros((48, 1024 // 128), dtype=torch.float16)
    assert "w has shape" in _raises(B.VG_ERR_SHAPE, vgm.verify_gemm_sign1, x, w, s1)
    _raises(B.VG_ERR_SHAPE, vgm.verify_gemm_affine2, x, w, s1, b)           # scales of the wrong group
    _raises(B.VG_ERR_SHAPE, vgm.verify_gemm_affine2, x, w, s, b[:40])       # biases of too few rows
    _raises(B.VG_ERR_DTYPE, vgm.verify_gemm_affine2, x, w, s.float(), b)    # scales not fp16
    _raises(B.VG_ERR_DTYPE, vgm.verify_gemm_affine2, x, w.long(), s, b)     # words not int32
    # biases None: scales must be the interleaved pairs [N, K/G, 2]
    assert "scales has shape" in _raises(B.VG_ERR_SHAPE, vgm.verify_gemm_affine2, x, w, s, None)
    sb = torch.zeros((48, 16, 2), dtype=torch.float16)
    _raises(B.VG_ERR_SHAPE, vgm.verify_gemm_affine2, x, w, sb, b)            # pairs beside biases
    _raises(B.VG_ERR_SHAPE, vgm.verify_gemm_affine2, x, w, sb[:, :8], None)  # pairs of the wrong group
    _raises(B.VG_ERR_DTYPE, vgm.verify_gemm_affine2, x, w, sb.float(), None)
    assert "GPU" in _raises(B.VG_ERR_ARG, vgm.verify_gemm_affine2, x, w, sb, None)   # valid: device check
    _raises(B.VG_ERR_SHAPE, vgm.pack_scale_bias, s, b[:, :8])                # shapes differ
    _raises(B.VG_ERR_DTYPE, vgm.pack_scale_bias, s.float(), b)
    assert "GPU" in _raises(B.VG_ERR_ARG, vgm.pack_scale_bias, s, b)
    _raises(B.VG_ERR_SHAPE, vgm.verify_gemm_affine2, x[:, :1000], w, s, b)  # K not a group multiple


def test_binding_checks_outputs_and_layout():
    torch = pytest.importorskip("torch")
    x, w, s, b = _affine2_tensors(torch)
    _raises(B.VG_ERR_SHAPE, vgm.verify_gemm_affine2, x, w, s, b, y=torch.zeros((1, 48)))  # too few rows
    _raises(B.VG_ERR_SHAPE, vgm.verify_gemm_affine2, x, w, s, b, y=torch.zeros((2, 47)))
    _raises(B.VG_ERR_DTYPE, vgm.verify_gemm_affine2, x, w, s, b, y=torch.zeros((2, 48), dtype=torch.float16))
    xt = torch.zeros((1024, 2), dtype=torch.float16).t()   # [2, 1024] view, not row-major
    assert "contiguous" in _raises(B.VG_ERR_SHAPE, vgm.verify_gemm_affine2, xt, w, s, b)
    wt = torch.zeros((64, 48), dtype=torch.int32).t()
    assert "contiguous" in _raises(B.VG_ERR_SHAPE, vgm.verify_gemm_affine2, x, wt, s, b)
    _raises(B.VG_ERR_SHAPE, vgm.verify_gemm_affine2, x[0], w, s, b)         # 1-D activations
    _raises(B.VG_ERR_DTYPE, vgm.verify_gemm_affine2, x.to(torch.int16), w, s, b)


def test_binding_refuses_host_tensors():
    torch = pytest.importorskip("torch")
    x, w, s, b = _affine2_tensors(torch)
    assert "GPU" in _raises(B.VG_ERR_ARG, vgm.verify_gemm_affine2, x, w, s, b)
    assert "GPU" in _raises(B.VG_ERR_ARG, vgm.verify_gemm_had2, x, w, s, b)
    assert "GPU" in _raises(B.VG_ERR_ARG, vgm.verify_argmax_rows, torch.zeros((2, 10)))
    assert "GPU" in _raises(B.VG_ERR_ARG, vgm.hadamard_rotate, x)


def test_binding_checks_argmax_experts_and_aux_arguments():
    torch = pytest.importorskip("torch")
    x, w, s, b = _affine2_tensors(torch, M=3)
    i32 = torch.int32
    _raises(B.VG_ERR_SHAPE, vgm.verify_gemm_argmax, "affine2", x, w, s, b, idx=torch.zeros(2, dtype=i32))
    _raises(B.VG_ERR_DTYPE, vgm.verify_gemm_argmax, "affine2", x, w, s, b, idx=torch.zeros(3, dtype=torch.int64))
    _raises(B.VG_ERR_SHAPE, vgm.verify_gemm_argmax, "affine2", x, w, s, b, idx=torch.zeros(3, dtype=i32),
            draft=torch.zeros(2, dtype=i32))
    _raises(B.VG_ERR_ARG, vgm.verify_gemm_argmax, "affine2", x, w, s, b, idx=torch.zeros(3, dtype=i32),
            accepted=torch.zeros(1, dtype=i32))
    _raises(B.VG_ERR_SHAPE, vgm.verify_gemm_had2, x, w, s, b, signs=torch.zeros(31, dtype=i32))
    # routed experts: w [E, N, words], route int32 [M, topk]
    we = torch.zeros((4, 48, 64), dtype=i32)
    se = torch.zeros((4, 48, 16), dtype=torch.float16)
    route = torch.zeros((3, 2), dtype=i32)
    _raises(B.VG_ERR_SHAPE, vgm.verify_gemm_experts, "affine2", x, route, w, s, b)          # 2-D weights
    _raises(B.VG_ERR_DTYPE, vgm.verify_gemm_experts, "affine2", x, route.long(), we, se, se)
    _raises(B.VG_ERR_SHAPE, vgm.verify_gemm_experts, "affine2", x, route[:2], we, se, se)
    _raises(B.VG_ERR_SHAPE, vgm.verify_gemm_experts, "affine2", x, route, we, se[:, :, :8], se)
    _raises(B.VG_ERR_SHAPE, vgm.verify_gemm_experts, "affine2", x, route, we, se, se,
            y=torch.zeros((3, 2, 47)))
    assert "GPU" in _raises(B.VG_ERR_ARG, vgm.verify_gemm_experts, "affine2", x, route, we, se, se)
    _raises(B.VG_ERR_SHAPE, vgm.verify_accept_greedy, torch.zeros((3, 10)), torch.zeros(2, dtype=i32))
    _raises(B.VG_ERR_DTYPE, vgm.verify_argmax_rows, torch.zeros((3, 10), dtype=torch.float16))
    _raises(B.VG_ERR_DTYPE, vgm.debug_unpack, "affine2", w, 1024, codes=torch.zeros((48, 1024), dtype=i32))
    _raises(B.VG_ERR_SHAPE, vgm.debug_unpack, "sign1", w, 1024)          # 2-bit words as 1-bit codes
    _raises(B.VG_ERR_SHAPE, vgm.stream_read, torch.zeros(16, dtype=i32), 128)


def test_debug_unpack_abi_validation():
    L = B.lib()
    assert L.vg_debug_unpack(9, B.VG_F16, ALIGNED, 4, 64, ALIGNED, None) == B.VG_ERR_ARG
    assert L.vg_debug_unpack(B.FMT_SIGN1, B.VG_F32, ALIGNED, 4, 64, ALIGNED, None) == B.VG_ERR_UNSUPPORTED
    assert L.vg_debug_unpack(B.FMT_SIGN1, 5, ALIGNED, 4, 64, ALIGNED, None) == B.VG_ERR_DTYPE
    assert L.vg_debug_unpack(B.FMT_SIGN1, B.VG_BF16, ALIGNED, 4, 48, ALIGNED, None) == B.VG_ERR_SHAPE
    assert L.vg_debug_unpack(B.FMT_AFFINE2, B.VG_F16, ALIGNED, 4, 40, ALIGNED, None) == B.VG_ERR_SHAPE
    assert L.vg_debug_unpack(B.FMT_AFFINE1, B.VG_BF16, ALIGNED + 4, 4, 64, ALIGNED, None) == B.VG_ERR_ALIGN
    assert L.vg_debug_unpack(B.FMT_HAD2, B.VG_F16, ALIGNED, 4, 64, None, None) == B.VG_ERR_ARG
