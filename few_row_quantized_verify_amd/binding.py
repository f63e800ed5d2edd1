"""ctypes binding of libverifygemm.so (argument marshalling only).

Every function takes device tensors, passes their pointers and the current HIP stream to
the C ABI declared in include/verify_gemm.h, and raises VerifyGemmError on a non-OK
status.  No step of the computation happens here; if the library is not built, import
of the library fails loudly (there is no fallback path).
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libverifygemm.so")

VG_OK, VG_ERR_ARG, VG_ERR_SHAPE, VG_ERR_ALIGN, VG_ERR_DTYPE, VG_ERR_UNSUPPORTED, VG_ERR_HIP = range(7)
STATUS_NAMES = ["VG_OK", "VG_ERR_ARG", "VG_ERR_SHAPE", "VG_ERR_ALIGN", "VG_ERR_DTYPE",
                "VG_ERR_UNSUPPORTED", "VG_ERR_HIP"]
VG_F32, VG_F16, VG_BF16 = 0, 1, 2
FMT_SIGN1, FMT_AFFINE2, FMT_HAD2, FMT_AFFINE1 = 0, 1, 2, 3
FORMATS = {"sign1": FMT_SIGN1, "affine2": FMT_AFFINE2, "had2": FMT_HAD2, "affine1": FMT_AFFINE1}
DTYPES = {"f32": VG_F32, "f16": VG_F16, "bf16": VG_BF16}


class VerifyGemmError(RuntimeError):
    def __init__(self, status: int, message: str):
        name = STATUS_NAMES[status] if 0 <= status < len(STATUS_NAMES) else str(status)
        super().__init__(f"{name}: {message}")
        self.status = status


_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int
_SIGS = {
    "verify_gemm_sign1": (_I, [_P, _I, _I, _I, _P, _P, _I, _P, _P]),
    "verify_gemm_affine1": (_I, [_P, _I, _I, _I, _P, _P, _P, _I, _P, _P]),
    "verify_gemm_had2_signed": (_I, [_P, _I, _I, _I, _P, _P, _P, _I, _I, _P, _P, _P]),
    "hadamard_rotate_signed": (_I, [_P, _I, _I, _I, _I, _P, _P, _P]),
    "verify_gemm_affine2": (_I, [_P, _I, _I, _I, _P, _P, _P, _I, _P, _P]),
    "verify_gemm_had2": (_I, [_P, _I, _I, _I, _P, _P, _P, _I, _I, _P, _P]),
    "hadamard_rotate": (_I, [_P, _I, _I, _I, _I, _P, _P]),
    "verify_argmax_rows": (_I, [_P, _I, _I, _P, _P]),
    "verify_accept_greedy": (_I, [_P, _I, _I, _P, _P, _P, _P]),
    "verify_gemm_argmax": (_I, [_I, _P, _I, _I, _I, _P, _P, _P, _I, _P, _P, _P, _P, _P]),
    "verify_gemm_argmax_noalloc": (_I, [_I, _P, _I, _I, _I, _P, _P, _P, _I, _P, _P, _P, _P, _P]),
    "verify_gemm_experts": (_I, [_I, _P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _I, _P, _P]),
    "vg_last_error": (ctypes.c_char_p, []),
    "vg_release_stream_workspace": (_I, [_P]),
    "vg_plan_variant": (_I, [_I, _I, _I, _I, _I]),
    "vg_variant_name": (ctypes.c_char_p, [_I]),
    "vg_force_variant": (_I, [_I]),
    "vg_variant_count": (_I, []),
    "vg_plan_ksplit": (_I, [_I, _I, _I, _I, _I]),
    "vg_force_ksplit": (_I, [_I]),
    "vg_plan_direct": (_I, [_I, _I, _I, _I, _I]),
    "vg_force_barrier_tail": (_I, [_I]),
    "vg_stream_read_blocks": (_I, []),
    "vg_stream_read": (_I, [_P, ctypes.c_size_t, _P, _P]),
    "vg_stream_read_config": (_I, [_P, ctypes.c_size_t, _P, _I, _I, _P]),
    "vg_debug_unpack": (_I, [_I, _I, _P, _I, _I, _P, _P]),
    "vg_debug_unpack_sign1": (_I, [_P, _I, _I, _P, _P]),
    "vg_debug_unpack_affine2": (_I, [_P, _I, _I, _P, _P]),
    "vg_pack_scale_bias": (_I, [_P, _P, ctypes.c_longlong, _P, _P]),
}


def lib() -> ctypes.CDLL:
    """Load the in-tree library once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m few_row_quantized_verify_amd.build`")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(l, name)
            fn.restype = res
            fn.argtypes = args
        _lib = l
    return _lib


def _check(status: int) -> None:
    if status != VG_OK:
        raise VerifyGemmError(status, lib().vg_last_error().decode())


def _torch():
    import torch
    return torch


def _stream(stream):
    """A HIP stream handle: None (torch's current stream), a torch stream, or a raw handle
    (int), which skips the current-stream lookup on hot call paths."""
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _xdtype(x) -> int:
    torch = _torch()
    try:
        return {torch.float32: VG_F32, torch.float16: VG_F16, torch.bfloat16: VG_BF16}[x.dtype]
    except KeyError:
        raise VerifyGemmError(VG_ERR_DTYPE, f"activation dtype {x.dtype} is not supported") from None


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _optr(t):
    """A device pointer, or NULL for None (the sign format's biases, or the interleaved
    scale-and-bias layout's)."""
    return ctypes.c_void_p(0) if t is None else ctypes.c_void_p(t.data_ptr())


# Elements per packed uint32 word and per quantization group of each format.
_WORD_K = {FMT_SIGN1: 32, FMT_AFFINE1: 32, FMT_AFFINE2: 16, FMT_HAD2: 16}
_GROUP = {FMT_SIGN1: 128, FMT_AFFINE1: 128, FMT_AFFINE2: 64, FMT_HAD2: 64}
_HAS_BIAS = {FMT_SIGN1: False, FMT_AFFINE1: True, FMT_AFFINE2: True, FMT_HAD2: True}


def _bad(status, msg):
    raise VerifyGemmError(status, msg)


def _tensor(t, name, shape, dtypes, dev=None):
    """The C ABI sees raw pointers only, so the binding checks what they point to: exact
    shape, dtype, row-major contiguity, and (last, so CPU-side checks come first) that the
    tensor lives on the same GPU as the activations."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        _bad(VG_ERR_ARG, f"{name} must be a torch tensor")
    if tuple(t.shape) != tuple(shape):
        _bad(VG_ERR_SHAPE, f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype not in dtypes:
        _bad(VG_ERR_DTYPE, f"{name} has dtype {t.dtype}, expected {' or '.join(str(d) for d in dtypes)}")
    if not t.is_contiguous():
        _bad(VG_ERR_SHAPE, f"{name} must be contiguous (row-major)")
    if dev is not None and t.device != dev:
        _bad(VG_ERR_ARG, f"{name} is on {t.device}, expected {dev}")
    return t


def _device(x):
    """The activations' device: a GPU, and the current one (the library launches there)."""
    torch = _torch()
    if not x.is_cuda:
        _bad(VG_ERR_ARG, f"x is on {x.device}, expected a GPU tensor")
    if x.device.index != torch.cuda.current_device():
        _bad(VG_ERR_ARG, f"x is on {x.device}, but the current device is cuda:{torch.cuda.current_device()}")
    return x.device


def _x(x):
    torch = _torch()
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        _bad(VG_ERR_SHAPE, "x must be a 2-D tensor [M, K]")
    _tensor(x, "x", x.shape, (torch.float32, torch.float16, torch.bfloat16))
    return x.shape


def _weights(fmt, w, scales, biases, N, K, lead=()):
    torch = _torch()
    wk, g = _WORD_K[fmt], _GROUP[fmt]
    if K % g:
        _bad(VG_ERR_SHAPE, f"K={K} is not a multiple of the group size {g}")
    _tensor(w, "w", (*lead, N, K // wk), (torch.int32,))
    if _HAS_BIAS[fmt] and biases is None:
        # the interleaved layout: each group's (scale, bias) pair side by side
        _tensor(scales, "scales", (*lead, N, K // g, 2), (torch.float16,))
        return
    _tensor(scales, "scales", (*lead, N, K // g), (torch.float16,))
    if _HAS_BIAS[fmt]:
        _tensor(biases, "biases", (*lead, N, K // g), (torch.float16,))


def _check_devices(dev, **tensors):
    for name, t in tensors.items():
        if t is not None and t.device != dev:
            _bad(VG_ERR_ARG, f"{name} is on {t.device}, expected {dev}")


def _out(y, M, N, x):
    torch = _torch()
    if y is None:
        return torch.empty((M, N), dtype=torch.float32, device=x.device)
    return _tensor(y, "y", (M, N), (torch.float32,))


def _gemm_args(fmt, x, w, scales, biases, y):
    """Validated (M, K, N, y) of a plain verify call."""
    torch = _torch()
    M, K = _x(x)
    if not isinstance(w, torch.Tensor) or w.dim() != 2:
        _bad(VG_ERR_SHAPE, "w must be a 2-D tensor [N, K / (codes per word)]")
    N = w.shape[0]
    _weights(fmt, w, scales, biases, N, K)
    if y is not None:
        _tensor(y, "y", (M, N), (torch.float32,))
    dev = _device(x)
    _check_devices(dev, w=w, scales=scales, biases=biases if _HAS_BIAS[fmt] else None, y=y)
    return M, K, N, _out(y, M, N, x)


def verify_gemm_sign1(x, wbits, scales, y=None, stream=None):
    """y[M, N] = x[M, K] @ W^T, W 1-bit sign g128 (wbits int32 [N, K/32], scales fp16 [N, K/128])."""
    M, K, N, y = _gemm_args(FMT_SIGN1, x, wbits, scales, None, y)
    _check(lib().verify_gemm_sign1(_ptr(x), _xdtype(x), M, K, _ptr(wbits), _ptr(scales), N,
                                   _ptr(y), _stream(stream)))
    return y


def verify_gemm_affine2(x, wq, scales, biases, y=None, stream=None):
    """y[M, N] = x[M, K] @ W^T, W 2-bit affine g64 (wq int32 [N, K/16], scales/biases fp16
    [N, K/64]; or biases None and scales the interleaved pairs [N, K/64, 2] of
    pack_scale_bias)."""
    M, K, N, y = _gemm_args(FMT_AFFINE2, x, wq, scales, biases, y)
    _check(lib().verify_gemm_affine2(_ptr(x), _xdtype(x), M, K, _ptr(wq), _ptr(scales),
                                     _optr(biases), N, _ptr(y), _stream(stream)))
    return y


def verify_gemm_affine1(x, wbits, scales, biases, y=None, stream=None):
    """y[M, N] = x[M, K] @ W^T, W MLX 1-bit affine g128 (wbits int32 [N, K/32], scales/biases
    fp16 [N, K/128]; or biases None and scales the interleaved pairs [N, K/128, 2])."""
    M, K, N, y = _gemm_args(FMT_AFFINE1, x, wbits, scales, biases, y)
    _check(lib().verify_gemm_affine1(_ptr(x), _xdtype(x), M, K, _ptr(wbits), _ptr(scales),
                                     _optr(biases), N, _ptr(y), _stream(stream)))
    return y


def verify_gemm_had2(x, wq, scales, biases, had_block=128, y=None, stream=None, signs=None):
    """y = ((x * D) @ blockdiag(H_B/sqrt(B))) @ W^T with W 2-bit affine g64, B = had_block;
    D = diag(+-1) from the sign bits `signs` (int32 [K/32], bit set: negate), or the
    identity when signs is None.  biases None: scales holds the interleaved pairs
    [N, K/64, 2]."""
    torch = _torch()
    if signs is not None:
        _tensor(signs, "signs", (_x(x)[1] // 32,), (torch.int32,))
    M, K, N, y = _gemm_args(FMT_HAD2, x, wq, scales, biases, y)
    _check_devices(x.device, signs=signs)
    if signs is None:
        _check(lib().verify_gemm_had2(_ptr(x), _xdtype(x), M, K, _ptr(wq), _ptr(scales),
                                      _optr(biases), N, had_block, _ptr(y), _stream(stream)))
    else:
        _check(lib().verify_gemm_had2_signed(_ptr(x), _xdtype(x), M, K, _ptr(wq), _ptr(scales),
                                             _optr(biases), N, had_block, _ptr(signs), _ptr(y),
                                             _stream(stream)))
    return y


def verify_gemm(fmt: str, x, w, scales, biases=None, y=None, stream=None):
    if fmt == "sign1":
        return verify_gemm_sign1(x, w, scales, y, stream)
    if fmt == "affine2":
        return verify_gemm_affine2(x, w, scales, biases, y, stream)
    if fmt == "had2":
        return verify_gemm_had2(x, w, scales, biases, 128, y, stream)
    if fmt == "affine1":
        return verify_gemm_affine1(x, w, scales, biases, y, stream)
    raise ValueError(fmt)


def verify_gemm_argmax(fmt: str, x, w, scales, biases=None, y=None, idx=None, draft=None, accepted=None,
                       stream=None):
    """The verify GEMM and the argmax of every output row in one call (the argmax fused into
    the GEMM where the plan allows).  Returns (y, idx), or (y, idx, accepted) when draft
    (int32 [M] on the device) is given."""
    torch = _torch()
    code = FORMATS[fmt]
    M = _x(x)[0]
    if idx is not None:
        _tensor(idx, "idx", (M,), (torch.int32,))
    if draft is not None:
        _tensor(draft, "draft", (M,), (torch.int32,))
    if accepted is not None:
        if draft is None:
            _bad(VG_ERR_ARG, "accepted needs draft")
        _tensor(accepted, "accepted", (1,), (torch.int32,))
    M, K, N, y = _gemm_args(code, x, w, scales, biases, y)
    _check_devices(x.device, idx=idx, draft=draft, accepted=accepted)
    if idx is None:
        idx = torch.empty((M,), dtype=torch.int32, device=x.device)
    if draft is not None and accepted is None:
        accepted = torch.empty((1,), dtype=torch.int32, device=x.device)
    null = ctypes.c_void_p(0)
    _check(lib().verify_gemm_argmax(code, _ptr(x), _xdtype(x), M, K, _ptr(w), _ptr(scales),
                                    null if biases is None else _ptr(biases), N, _ptr(y), _ptr(idx),
                                    null if draft is None else _ptr(draft),
                                    null if accepted is None else _ptr(accepted), _stream(stream)))
    return (y, idx) if draft is None else (y, idx, accepted)


def verify_gemm_argmax_noalloc(fmt: str, x, w, scales, biases, y, idx=None, draft=None, accepted=None,
                               stream=None):
    """verify_gemm_argmax with the library's static scratch: nothing is allocated, by the
    library or here, so y (and idx, and accepted with draft) must be given.  With idx None
    only y is computed.  Returns y, (y, idx) or (y, idx, accepted) like the allocating call."""
    torch = _torch()
    code = FORMATS[fmt]
    M = _x(x)[0]
    if y is None:
        _bad(VG_ERR_ARG, "y must be given: this call allocates nothing")
    if idx is not None:
        _tensor(idx, "idx", (M,), (torch.int32,))
    if (draft is None) != (accepted is None):
        _bad(VG_ERR_ARG, "draft and accepted go together")
    if draft is not None:
        if idx is None:
            _bad(VG_ERR_ARG, "draft needs idx")
        _tensor(draft, "draft", (M,), (torch.int32,))
        _tensor(accepted, "accepted", (1,), (torch.int32,))
    M, K, N, y = _gemm_args(code, x, w, scales, biases, y)
    _check_devices(x.device, idx=idx, draft=draft, accepted=accepted)
    null = ctypes.c_void_p(0)
    _check(lib().verify_gemm_argmax_noalloc(code, _ptr(x), _xdtype(x), M, K, _ptr(w), _ptr(scales),
                                            null if biases is None else _ptr(biases), N, _ptr(y),
                                            null if idx is None else _ptr(idx),
                                            null if draft is None else _ptr(draft),
                                            null if accepted is None else _ptr(accepted), _stream(stream)))
    if idx is None:
        return y
    return (y, idx) if draft is None else (y, idx, accepted)


def verify_gemm_experts(fmt: str, x, route, w, scales, biases=None, y=None, stream=None):
    """Grouped routed-expert verify: y[m, s] = x[m] @ W_e^T with e = route[m, s] (int32
    [M, topk] on the device, values outside 0..E-1 mark unused slots, whose rows of y are
    not written).  w, scales, biases: the E experts' packed weights stacked on dim 0.
    Returns y, fp32 [M, topk, N]."""
    torch = _torch()
    code = FORMATS[fmt]
    M, K = _x(x)
    if not isinstance(route, torch.Tensor) or route.dim() != 2:
        _bad(VG_ERR_SHAPE, "route must be a 2-D tensor [M, topk]")
    if not isinstance(w, torch.Tensor) or w.dim() != 3:
        _bad(VG_ERR_SHAPE, "w must be a 3-D tensor [E, N, K / (codes per word)]")
    topk = route.shape[1]
    E, N = w.shape[0], w.shape[1]
    _tensor(route, "route", (M, topk), (torch.int32,))
    _weights(code, w, scales, biases, N, K, lead=(E,))
    if y is not None:
        _tensor(y, "y", (M, topk, N), (torch.float32,))
    dev = _device(x)
    _check_devices(dev, route=route, w=w, scales=scales, biases=biases if _HAS_BIAS[code] else None, y=y)
    if y is None:
        y = torch.empty((M, topk, N), dtype=torch.float32, device=x.device)
    b = ctypes.c_void_p(0) if biases is None else _ptr(biases)
    _check(lib().verify_gemm_experts(code, _ptr(x), _xdtype(x), M, K, E, topk, _ptr(route),
                                     _ptr(w), _ptr(scales), b, N, _ptr(y), _stream(stream)))
    return y


def hadamard_rotate(x, block=128, out=None, stream=None, signs=None):
    torch = _torch()
    M, K = _x(x)
    if out is not None:
        _tensor(out, "out", (M, K), (torch.float32,))
    if signs is not None:
        _tensor(signs, "signs", (K // 32,), (torch.int32,))
    dev = _device(x)
    _check_devices(dev, out=out, signs=signs)
    if out is None:
        out = torch.empty((M, K), dtype=torch.float32, device=x.device)
    if signs is None:
        _check(lib().hadamard_rotate(_ptr(x), _xdtype(x), M, K, block, _ptr(out), _stream(stream)))
    else:
        _check(lib().hadamard_rotate_signed(_ptr(x), _xdtype(x), M, K, block, _ptr(signs), _ptr(out),
                                            _stream(stream)))
    return out


def _logits(y):
    torch = _torch()
    if not isinstance(y, torch.Tensor) or y.dim() != 2:
        _bad(VG_ERR_SHAPE, "y must be a 2-D tensor [M, N]")
    _tensor(y, "y", y.shape, (torch.float32,))
    return y.shape


def verify_argmax_rows(y, idx=None, stream=None):
    torch = _torch()
    M, N = _logits(y)
    if idx is not None:
        _tensor(idx, "idx", (M,), (torch.int32,))
    dev = _device(y)
    _check_devices(dev, idx=idx)
    if idx is None:
        idx = torch.empty((M,), dtype=torch.int32, device=y.device)
    _check(lib().verify_argmax_rows(_ptr(y), M, N, _ptr(idx), _stream(stream)))
    return idx


def verify_accept_greedy(y, draft, idx=None, accepted=None, stream=None):
    """(idx, accepted): per-row argmax of the logits y [M, N] and the number of leading rows
    whose argmax equals draft[m] (draft: int32 [M] on the device)."""
    torch = _torch()
    M, N = _logits(y)
    _tensor(draft, "draft", (M,), (torch.int32,))
    if idx is not None:
        _tensor(idx, "idx", (M,), (torch.int32,))
    if accepted is not None:
        _tensor(accepted, "accepted", (1,), (torch.int32,))
    dev = _device(y)
    _check_devices(dev, draft=draft, idx=idx, accepted=accepted)
    if idx is None:
        idx = torch.empty((M,), dtype=torch.int32, device=y.device)
    if accepted is None:
        accepted = torch.empty((1,), dtype=torch.int32, device=y.device)
    _check(lib().verify_accept_greedy(_ptr(y), M, N, _ptr(draft), _ptr(idx), _ptr(accepted), _stream(stream)))
    return idx, accepted


def pack_scale_bias(scales, biases, out=None, stream=None):
    """The interleaved scale-and-bias layout of an affine format's group metadata, built on
    the device once when the weights are loaded: scales and biases fp16 [..., G] (same
    shape) give out fp16 [..., G, 2] with out[..., 0] = scales and out[..., 1] = biases.
    Pass it as `scales` with biases None to any affine verify call."""
    torch = _torch()
    if not isinstance(scales, torch.Tensor) or not isinstance(biases, torch.Tensor):
        _bad(VG_ERR_ARG, "scales and biases must be torch tensors")
    _tensor(scales, "scales", scales.shape, (torch.float16,))
    _tensor(biases, "biases", scales.shape, (torch.float16,))
    if not scales.is_cuda:
        _bad(VG_ERR_ARG, f"scales is on {scales.device}, expected a GPU tensor")
    _check_devices(scales.device, biases=biases)
    if out is None:
        out = torch.empty((*scales.shape, 2), dtype=torch.float16, device=scales.device)
    _tensor(out, "out", (*scales.shape, 2), (torch.float16,), scales.device)
    _check(lib().vg_pack_scale_bias(_ptr(scales), _ptr(biases), scales.numel(), _ptr(out), _stream(stream)))
    return out


def stream_read(buf, nbytes: int, sink=None, stream=None, loads_in_flight: int = 4, wgs_per_cu: int = 8):
    """Measurement aid: read nbytes of the device tensor buf once (vg_stream_read_config)."""
    torch = _torch()
    if not isinstance(buf, torch.Tensor) or not buf.is_contiguous():
        _bad(VG_ERR_ARG, "buf must be a contiguous tensor")
    if nbytes > buf.numel() * buf.element_size():
        _bad(VG_ERR_SHAPE, f"nbytes={nbytes} exceeds the buffer's {buf.numel() * buf.element_size()} bytes")
    if sink is None:
        sink = torch.empty((lib().vg_stream_read_blocks(),), dtype=torch.int32, device=buf.device)
    _tensor(sink, "sink", (lib().vg_stream_read_blocks(),), (torch.int32,))
    dev = _device(buf)
    _check_devices(dev, sink=sink)
    _check(lib().vg_stream_read_config(_ptr(buf), nbytes, _ptr(sink), loads_in_flight, wgs_per_cu,
                                       _stream(stream)))
    return sink


def debug_unpack(fmt: str, w, K, codes=None, stream=None, x_dtype: str = "f16"):
    """Codes uint8 [N, K] decoded by the GEMM's register decode for (fmt, x_dtype)."""
    torch = _torch()
    code = FORMATS[fmt]
    if not isinstance(w, torch.Tensor) or w.dim() != 2:
        _bad(VG_ERR_SHAPE, "w must be a 2-D tensor [N, K / (codes per word)]")
    N = w.shape[0]
    if K % _WORD_K[code]:
        _bad(VG_ERR_SHAPE, f"K={K} is not a multiple of {_WORD_K[code]}")
    _tensor(w, "w", (N, K // _WORD_K[code]), (torch.int32,))
    if codes is not None:
        _tensor(codes, "codes", (N, K), (torch.uint8,))
    dev = _device(w)
    _check_devices(dev, codes=codes)
    if codes is None:
        codes = torch.empty((N, K), dtype=torch.uint8, device=w.device)
    _check(lib().vg_debug_unpack(code, DTYPES[x_dtype], _ptr(w), N, K, _ptr(codes), _stream(stream)))
    return codes


def release_stream_workspace(stream=None) -> None:
    """Free the library's workspace of a stream (torch's current stream by default)."""
    _check(lib().vg_release_stream_workspace(_stream(stream)))


def plan_variant(fmt: str, x_dtype: str, M: int, N: int, K: int) -> int:
    return lib().vg_plan_variant(FORMATS[fmt], DTYPES[x_dtype], M, N, K)


def variant_name(v: int) -> str:
    return lib().vg_variant_name(v).decode()


def variant_count() -> int:
    return lib().vg_variant_count()


def force_variant(v: int) -> None:
    _check(lib().vg_force_variant(v))


def plan_ksplit(fmt: str, x_dtype: str, M: int, N: int, K: int) -> int:
    return lib().vg_plan_ksplit(FORMATS[fmt], DTYPES[x_dtype], M, N, K)


def force_ksplit(ks: int) -> None:
    _check(lib().vg_force_ksplit(ks))


def plan_direct(fmt: str, x_dtype: str, M: int, N: int, K: int) -> int:
    """1 when a plain verify call stores each tile from the wave that completes it (no
    barrier after the main loop), 0 when it finishes the tiles after a barrier, -1 when no
    call takes the arguments."""
    return lib().vg_plan_direct(FORMATS[fmt], DTYPES[x_dtype], M, N, K)


def force_barrier_tail(on: bool) -> None:
    """Make later MFMA calls finish every tile after the workgroup barrier (tests)."""
    _check(lib().vg_force_barrier_tail(1 if on else 0))
