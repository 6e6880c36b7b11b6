"""MI355X (gfx950) microscaled convolution: MicroQonv's training hot path.

Thin Python binding over the C ABI of libmqconv.so (include/mqconv.h). Every
function has the C entry point's name and only marshals arguments: torch
tensors provide device memory and the stream, all arithmetic runs in the HIP
kernels. Importing this package does not load the library; the first call
does, and raises if it has not been built.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional, Sequence, Tuple, Union

_HERE = os.path.dirname(os.path.abspath(__file__))
# MQCONV_LIB names another build of the same library (the host-sanitizer
# build of the tests); there is no fallback if it is missing
LIB_PATH = os.environ.get("MQCONV_LIB") or os.path.join(_HERE, "libmqconv.so")

MQ_OK = 0
MQ_ERR_SHAPE = -2
STATUS_NAMES = {0: "MQ_OK", -1: "MQ_ERR_NULL", -2: "MQ_ERR_SHAPE", -3: "MQ_ERR_FORMAT",
                -4: "MQ_ERR_ALIGN", -5: "MQ_ERR_WORKSPACE", -6: "MQ_ERR_UNSUPPORTED", -7: "MQ_ERR_HIP"}
E4M3, E5M2, E2M3, E3M2, E2M1 = 0, 1, 2, 3, 4
ROLE_ACT, ROLE_WEIGHT, ROLE_GRAD = 0, 1, 2
OP_FWD, OP_DGRAD, OP_WGRAD = 0, 1, 2


class MqConvError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str = ""):
        self.status = status
        msg = f"{where}: {STATUS_NAMES.get(status, status)}"
        super().__init__(msg + (f" ({detail})" if detail else f" ({_status_string(status)})"))


class mq_conv(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("n", "cin", "h", "w", "cout", "kh", "kw", "stride_h", "stride_w", "pad_h", "pad_w")]


class mq_mx(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("fmt", ctypes.c_int),
                ("block_partner", ctypes.c_int32), ("role", ctypes.c_int),
                ("d0", ctypes.c_int32), ("d1", ctypes.c_int32), ("d2", ctypes.c_int32),
                ("d3", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libmqconv.so (raises if it is missing: there is no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run microscaling_quantized_convolution_mxq_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        P, S, I, I32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int32
        CV = ctypes.POINTER(mq_conv)
        sig = {
            "mqconv_abi_version": (I, []),
            "mqconv_status_string": (ctypes.c_char_p, [I]),
            "mqconv_inject_launch_failure": (I, [I]),
            "mqconv_codes_bytes": (S, [I, I, I32, I32, I32, I32]),
            "mqconv_scales_bytes": (S, [I, I32, I32, I32, I32, I32]),
            "mqconv_im2col_codes_bytes": (S, [CV, I]),
            "mqconv_im2col_scales_bytes": (S, [CV, I32]),
            "mqconv_quantize": (I, [P, mq_mx, P]),
            "mqconv_quantize_group": (I, [I32, P, ctypes.POINTER(mq_mx), P]),
            "mqconv_quantize_sr": (I, [P, mq_mx, ctypes.c_uint64, P]),
            "mqconv_cbf_im2col": (I, [CV, mq_mx, P, P, P]),
            "mqconv_workspace_bytes": (S, [CV, I, I, I]),
            "mqconv_forward": (I, [CV, mq_mx, mq_mx, P, P, S, P]),
            "mqconv_forward_mx": (I, [CV, mq_mx, mq_mx, mq_mx, P, S, P]),
            "mqconv_backward_data": (I, [CV, mq_mx, mq_mx, P, P, S, P]),
            "mqconv_backward_data_mx": (I, [CV, mq_mx, mq_mx, mq_mx, P, S, P]),
            "mqconv_backward_weight": (I, [CV, mq_mx, mq_mx, P, P, S, P]),
            "mqconv_backward_weight_noalloc": (I, [CV, mq_mx, mq_mx, P, P]),
            "mqconv_naive_workspace_bytes": (S, [CV, I, I, I]),
            "mqconv_nvfp_scales_bytes": (S, [I, I32, I32, I32, I32]),
            "mqconv_nvfp_workspace_bytes": (S, []),
            "mqconv_nvfp_quantize": (I, [P, I, I, I32, I32, I32, I32, P, P, P, P, S, P]),
            "mqconv_cuyckens_col_codes_bytes": (S, [CV, I]),
            "mqconv_cuyckens_col_scales_bytes": (S, [CV]),
            "mqconv_cuyckens_workspace_bytes": (S, [CV, I, I, I]),
            "mqconv_cuyckens_im2col_quantize": (I, [CV, P, I, P, P, P]),
            "mqconv_cuyckens_forward": (I, [CV, P, P, I, P, I, P, P, S, P]),
            "mqconv_cuyckens_backward_data": (I, [CV, P, P, I, I, P, P, S, P]),
            "mqconv_cuyckens_backward_weight": (I, [CV, P, P, P, I, I, P, P, S, P]),
            "mqconv_naive_forward": (I, [CV, P, P, I, I, P, P, S, P]),
            "mqconv_naive_backward_data": (I, [CV, P, P, I, I, P, P, S, P]),
            "mqconv_naive_backward_weight": (I, [CV, P, P, I, I, P, P, S, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


EXPORTED = ("mqconv_abi_version", "mqconv_status_string", "mqconv_inject_launch_failure", "mqconv_codes_bytes", "mqconv_scales_bytes",
            "mqconv_im2col_codes_bytes", "mqconv_im2col_scales_bytes", "mqconv_quantize", "mqconv_quantize_group",
            "mqconv_quantize_sr",
            "mqconv_cbf_im2col", "mqconv_workspace_bytes", "mqconv_forward", "mqconv_forward_mx", "mqconv_backward_data",
            "mqconv_backward_data_mx", "mqconv_backward_weight", "mqconv_backward_weight_noalloc",
            "mqconv_naive_workspace_bytes", "mqconv_naive_forward",
            "mqconv_naive_backward_data", "mqconv_naive_backward_weight", "mqconv_nvfp_scales_bytes",
            "mqconv_nvfp_workspace_bytes", "mqconv_nvfp_quantize", "mqconv_cuyckens_col_codes_bytes",
            "mqconv_cuyckens_col_scales_bytes", "mqconv_cuyckens_workspace_bytes", "mqconv_cuyckens_im2col_quantize",
            "mqconv_cuyckens_forward", "mqconv_cuyckens_backward_data", "mqconv_cuyckens_backward_weight")


def _status_string(status: int) -> str:
    try:
        return lib().mqconv_status_string(status).decode()
    except Exception:  # pragma: no cover - only while formatting an error
        return "?"


def _check(status: int, where: str) -> None:
    if status != MQ_OK:
        raise MqConvError(status, where)


def _conv(shape) -> mq_conv:
    t = shape.as_tuple() if hasattr(shape, "as_tuple") else tuple(shape)
    return mq_conv(*t)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    return t.data_ptr() if hasattr(t, "data_ptr") else int(t)


def _buf(t, nbytes: int, dtype: Optional[str], what: str) -> Optional[int]:
    """Device address of a buffer handed to the library. A torch tensor must
    be contiguous, of the expected dtype (None: any), hold at least `nbytes`
    bytes and live on the GPU, else MqConvError(MQ_ERR_SHAPE) is raised before
    the C call: the C side sees raw pointers and cannot check any of this. A
    plain integer address is passed through unchecked (the caller vouches for
    it)."""
    if t is None or not hasattr(t, "data_ptr"):
        return _ptr(t)
    if dtype is not None and str(t.dtype) != "torch." + dtype:
        raise MqConvError(MQ_ERR_SHAPE, what, f"dtype {t.dtype}, expected torch.{dtype}")
    if not t.is_contiguous():
        raise MqConvError(MQ_ERR_SHAPE, what, "tensor is not contiguous")
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise MqConvError(MQ_ERR_SHAPE, what, f"{have} bytes, needs {nbytes}")
    if not t.is_cuda:
        raise MqConvError(MQ_ERR_SHAPE, what, "not a GPU tensor")
    return t.data_ptr()


def _f32(t, count: int, what: str) -> Optional[int]:
    return _buf(t, 4 * count, "float32", what)


def _dims(shape):
    """(n, cin, h, w, cout, kh, kw, ho, wo) of a convolution."""
    c = _conv(shape)
    ho = (c.h + 2 * c.pad_h - c.kh) // c.stride_h + 1 if c.stride_h > 0 else 0
    wo = (c.w + 2 * c.pad_w - c.kw) // c.stride_w + 1 if c.stride_w > 0 else 0
    return c.n, c.cin, c.h, c.w, c.cout, c.kh, c.kw, max(ho, 0), max(wo, 0)


def _nx(shape):
    n, cin, h, w, *_ = _dims(shape)
    return h * w * n * cin


def _nw(shape):
    _, cin, _, _, cout, kh, kw, _, _ = _dims(shape)
    return cout * kh * kw * cin


def _ny(shape):
    n, _, _, _, cout, _, _, ho, wo = _dims(shape)
    return ho * wo * n * cout


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


@dataclasses.dataclass
class MxTensor:
    """A packed MX tensor on the device (layouts in include/mqconv.h)."""
    codes: object  # torch.uint8 tensor
    scales: object  # torch.uint8 tensor
    fmt: int
    bp: int
    role: int
    dims: Tuple[int, int, int, int]

    @staticmethod
    def empty(role: int, fmt: int, bp: int, dims: Sequence[int], device="cuda") -> "MxTensor":
        import torch
        nc = mqconv_codes_bytes(role, fmt, *dims)
        ns = mqconv_scales_bytes(role, bp, *dims)
        if nc == 0 or ns == 0:
            raise MqConvError(-2, "MxTensor.empty")
        return MxTensor(torch.empty(nc, dtype=torch.uint8, device=device),
                        torch.empty(ns, dtype=torch.uint8, device=device), fmt, bp, role, tuple(dims))

    def c_struct(self, what: str = "MxTensor") -> mq_mx:
        """The C view; tensor buffers are checked against the sizes the
        layout needs (invalid role/format/dims are left to the C call, which
        reports them with its own status)."""
        nc = mqconv_codes_bytes(self.role, self.fmt, *self.dims)
        ns = mqconv_scales_bytes(self.role, self.bp, *self.dims)
        return mq_mx(_buf(self.codes, nc, "uint8", what + ".codes"), _buf(self.scales, ns, "uint8", what + ".scales"),
                     self.fmt, self.bp, self.role, *self.dims)


def mqconv_abi_version() -> int:
    return lib().mqconv_abi_version()


def mqconv_inject_launch_failure(n: int) -> None:
    """The n-th launch check from now reports a launch failure (n = 0: none);
    for tests of the error paths."""
    _check(lib().mqconv_inject_launch_failure(int(n)), "mqconv_inject_launch_failure")


def mqconv_status_string(status: int) -> str:
    return _status_string(status)


def mqconv_codes_bytes(role: int, fmt: int, d0: int, d1: int, d2: int, d3: int) -> int:
    return lib().mqconv_codes_bytes(role, fmt, d0, d1, d2, d3)


def mqconv_scales_bytes(role: int, bp: int, d0: int, d1: int, d2: int, d3: int) -> int:
    return lib().mqconv_scales_bytes(role, bp, d0, d1, d2, d3)


def mqconv_im2col_codes_bytes(shape, fmt: int) -> int:
    return lib().mqconv_im2col_codes_bytes(ctypes.byref(_conv(shape)), fmt)


def mqconv_im2col_scales_bytes(shape, bp: int) -> int:
    return lib().mqconv_im2col_scales_bytes(ctypes.byref(_conv(shape)), bp)


def _prod(d):
    r = 1
    for v in d:
        r *= int(v)
    return r


def mqconv_quantize(src, dst: MxTensor, stream=None) -> None:
    _check(lib().mqconv_quantize(_f32(src, _prod(dst.dims), "src"), dst.c_struct("dst"), _stream(stream)),
           "mqconv_quantize")


def mqconv_quantize_sr(src, dst: MxTensor, seed: int, stream=None) -> None:
    """mqconv_quantize with stochastically rounded elements (random words from seed)."""
    _check(lib().mqconv_quantize_sr(_f32(src, _prod(dst.dims), "src"), dst.c_struct("dst"), int(seed) & (2**64 - 1),
                                    _stream(stream)), "mqconv_quantize_sr")


QUANTIZE_GROUP_MAX = 8


def mqconv_quantize_group(pairs, stream=None) -> None:
    """mqconv_quantize of several (src, dst MxTensor) pairs in one call."""
    pairs = list(pairs)
    n = len(pairs)
    srcs = (ctypes.c_void_p * max(1, n))(*[_f32(p[0], _prod(p[1].dims), f"src[{i}]") for i, p in enumerate(pairs)])
    dsts = (mq_mx * max(1, n))(*[p[1].c_struct(f"dst[{i}]") for i, p in enumerate(pairs)])
    _check(lib().mqconv_quantize_group(n, srcs, dsts, _stream(stream)), "mqconv_quantize_group")


def mqconv_cbf_im2col(shape, xq: MxTensor, col_codes, col_scales, stream=None) -> None:
    cc = _buf(col_codes, mqconv_im2col_codes_bytes(shape, xq.fmt), "uint8", "col_codes")
    cs = _buf(col_scales, mqconv_im2col_scales_bytes(shape, xq.bp), "uint8", "col_scales")
    _check(lib().mqconv_cbf_im2col(ctypes.byref(_conv(shape)), xq.c_struct("xq"), cc, cs, _stream(stream)),
           "mqconv_cbf_im2col")


def mqconv_workspace_bytes(shape, op: int, fa: int, fb: int) -> int:
    return lib().mqconv_workspace_bytes(ctypes.byref(_conv(shape)), op, fa, fb)


def _ws(ws):
    """(address, bytes) of a workspace; its size is checked by the C call."""
    if ws is None:
        return None, 0
    if not hasattr(ws, "data_ptr"):
        raise MqConvError(MQ_ERR_SHAPE, "ws", "a workspace must be a tensor (its size is passed on)")
    return _buf(ws, 0, None, "ws"), ws.numel() * ws.element_size()


def mqconv_forward(shape, xq: MxTensor, wq: MxTensor, y, ws=None, stream=None) -> None:
    p, n = _ws(ws)
    _check(lib().mqconv_forward(ctypes.byref(_conv(shape)), xq.c_struct("xq"), wq.c_struct("wq"),
                                _f32(y, _ny(shape), "y"), p, n, _stream(stream)), "mqconv_forward")


def mqconv_forward_mx(shape, xq: MxTensor, wq: MxTensor, yq: MxTensor, ws=None, stream=None) -> None:
    p, n = _ws(ws)
    _check(lib().mqconv_forward_mx(ctypes.byref(_conv(shape)), xq.c_struct("xq"), wq.c_struct("wq"),
                                   yq.c_struct("yq"), p, n, _stream(stream)), "mqconv_forward_mx")


def mqconv_backward_data(shape, dyq: MxTensor, wq: MxTensor, dx, ws=None, stream=None) -> None:
    p, n = _ws(ws)
    _check(lib().mqconv_backward_data(ctypes.byref(_conv(shape)), dyq.c_struct("dyq"), wq.c_struct("wq"),
                                      _f32(dx, _nx(shape), "dx"), p, n, _stream(stream)), "mqconv_backward_data")


def mqconv_backward_data_mx(shape, dyq: MxTensor, wq: MxTensor, dxq: MxTensor, ws=None, stream=None) -> None:
    p, n = _ws(ws)
    _check(lib().mqconv_backward_data_mx(ctypes.byref(_conv(shape)), dyq.c_struct("dyq"), wq.c_struct("wq"),
                                         dxq.c_struct("dxq"), p, n, _stream(stream)), "mqconv_backward_data_mx")


def mqconv_backward_weight(shape, dyq: MxTensor, xq: MxTensor, dw, ws=None, stream=None) -> None:
    p, n = _ws(ws)
    _check(lib().mqconv_backward_weight(ctypes.byref(_conv(shape)), dyq.c_struct("dyq"), xq.c_struct("xq"),
                                        _f32(dw, _nw(shape), "dw"), p, n, _stream(stream)), "mqconv_backward_weight")


# scratch bytes the library holds per device for mqconv_backward_weight_noalloc
NOALLOC_SCRATCH_BYTES = 96 << 20


def mqconv_backward_weight_noalloc(shape, dyq: MxTensor, xq: MxTensor, dw, stream=None) -> None:
    """mqconv_backward_weight with the library's own per-device scratch array
    instead of a workspace (no allocation anywhere in the call)."""
    _check(lib().mqconv_backward_weight_noalloc(ctypes.byref(_conv(shape)), dyq.c_struct("dyq"), xq.c_struct("xq"),
                                                _f32(dw, _nw(shape), "dw"), _stream(stream)),
           "mqconv_backward_weight_noalloc")


def mqconv_naive_workspace_bytes(shape, op: int, fa: int, fb: int) -> int:
    return lib().mqconv_naive_workspace_bytes(ctypes.byref(_conv(shape)), op, fa, fb)


def mqconv_naive_forward(shape, x, w, fx: int, fw: int, y, ws, stream=None) -> None:
    p, n = _ws(ws)
    _check(lib().mqconv_naive_forward(ctypes.byref(_conv(shape)), _f32(x, _nx(shape), "x"), _f32(w, _nw(shape), "w"),
                                      fx, fw, _f32(y, _ny(shape), "y"), p, n, _stream(stream)),
           "mqconv_naive_forward")


def mqconv_naive_backward_data(shape, dy, w, fdy: int, fw: int, dx, ws, stream=None) -> None:
    p, n = _ws(ws)
    _check(lib().mqconv_naive_backward_data(ctypes.byref(_conv(shape)), _f32(dy, _ny(shape), "dy"),
                                            _f32(w, _nw(shape), "w"), fdy, fw, _f32(dx, _nx(shape), "dx"), p, n,
                                            _stream(stream)), "mqconv_naive_backward_data")


def mqconv_naive_backward_weight(shape, dy, x, fdy: int, fx: int, dw, ws, stream=None) -> None:
    p, n = _ws(ws)
    _check(lib().mqconv_naive_backward_weight(ctypes.byref(_conv(shape)), _f32(dy, _ny(shape), "dy"),
                                              _f32(x, _nx(shape), "x"), fdy, fx, _f32(dw, _nw(shape), "dw"), p, n,
                                              _stream(stream)), "mqconv_naive_backward_weight")


# ---- square-block comparator (include/mqconv.h) ----------------------------------
def mqconv_cuyckens_col_codes_bytes(shape, fx: int) -> int:
    return lib().mqconv_cuyckens_col_codes_bytes(ctypes.byref(_conv(shape)), fx)


def mqconv_cuyckens_col_scales_bytes(shape) -> int:
    return lib().mqconv_cuyckens_col_scales_bytes(ctypes.byref(_conv(shape)))


def mqconv_cuyckens_workspace_bytes(shape, op: int, fa: int, fb: int) -> int:
    return lib().mqconv_cuyckens_workspace_bytes(ctypes.byref(_conv(shape)), op, fa, fb)


def mqconv_cuyckens_im2col_quantize(shape, x, fx: int, col_codes, col_scales, stream=None) -> None:
    cc = _buf(col_codes, mqconv_cuyckens_col_codes_bytes(shape, fx), "uint8", "col_codes")
    cs = _buf(col_scales, mqconv_cuyckens_col_scales_bytes(shape), "uint8", "col_scales")
    _check(lib().mqconv_cuyckens_im2col_quantize(ctypes.byref(_conv(shape)), _f32(x, _nx(shape), "x"), fx, cc, cs,
                                                 _stream(stream)), "mqconv_cuyckens_im2col_quantize")


def mqconv_cuyckens_forward(shape, col_codes, col_scales, fx: int, w, fw: int, y, ws, stream=None) -> None:
    p, n = _ws(ws)
    cc = _buf(col_codes, mqconv_cuyckens_col_codes_bytes(shape, fx), "uint8", "col_codes")
    cs = _buf(col_scales, mqconv_cuyckens_col_scales_bytes(shape), "uint8", "col_scales")
    _check(lib().mqconv_cuyckens_forward(ctypes.byref(_conv(shape)), cc, cs, fx, _f32(w, _nw(shape), "w"), fw,
                                         _f32(y, _ny(shape), "y"), p, n, _stream(stream)), "mqconv_cuyckens_forward")


def mqconv_cuyckens_backward_data(shape, dy, w, fdy: int, fw: int, dx, ws, stream=None) -> None:
    p, n = _ws(ws)
    _check(lib().mqconv_cuyckens_backward_data(ctypes.byref(_conv(shape)), _f32(dy, _ny(shape), "dy"),
                                               _f32(w, _nw(shape), "w"), fdy, fw, _f32(dx, _nx(shape), "dx"), p, n,
                                               _stream(stream)), "mqconv_cuyckens_backward_data")


def mqconv_cuyckens_backward_weight(shape, dy, col_codes, col_scales, fdy: int, fx: int, dw, ws, stream=None) -> None:
    p, n = _ws(ws)
    cc = _buf(col_codes, mqconv_cuyckens_col_codes_bytes(shape, fx), "uint8", "col_codes")
    cs = _buf(col_scales, mqconv_cuyckens_col_scales_bytes(shape), "uint8", "col_scales")
    _check(lib().mqconv_cuyckens_backward_weight(ctypes.byref(_conv(shape)), _f32(dy, _ny(shape), "dy"), cc, cs, fdy,
                                                 fx, _f32(dw, _nw(shape), "dw"), p, n, _stream(stream)),
           "mqconv_cuyckens_backward_weight")


# ---- two-level (NVFP-style) quantization (include/mqconv.h) -------------------------
def mqconv_nvfp_scales_bytes(role: int, d0: int, d1: int, d2: int, d3: int) -> int:
    return lib().mqconv_nvfp_scales_bytes(role, d0, d1, d2, d3)


def mqconv_nvfp_workspace_bytes() -> int:
    return lib().mqconv_nvfp_workspace_bytes()


def mqconv_nvfp_quantize(src, role: int, fmt: int, dims, codes, block_scales, tensor_scale, ws, stream=None) -> None:
    """Two-level quantization of the fp32 tensor src (role layout, dims) into
    packed codes, E4M3 block scales and one fp32 tensor scale (device)."""
    d = tuple(int(v) for v in dims)
    p, n = _ws(ws)
    _check(lib().mqconv_nvfp_quantize(_f32(src, _prod(d), "src"), role, fmt, *d,
                                      _buf(codes, mqconv_codes_bytes(role, fmt, *d), "uint8", "codes"),
                                      _buf(block_scales, mqconv_nvfp_scales_bytes(role, *d), "uint8", "block_scales"),
                                      _f32(tensor_scale, 1, "tensor_scale"), p, n, _stream(stream)),
           "mqconv_nvfp_quantize")
