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
LIB_PATH = os.path.join(_HERE, "libmqconv.so")

MQ_OK = 0
STATUS_NAMES = {0: "MQ_OK", -1: "MQ_ERR_NULL", -2: "MQ_ERR_SHAPE", -3: "MQ_ERR_FORMAT",
                -4: "MQ_ERR_ALIGN", -5: "MQ_ERR_WORKSPACE", -6: "MQ_ERR_UNSUPPORTED", -7: "MQ_ERR_HIP"}
E4M3, E5M2, E2M3, E3M2, E2M1 = 0, 1, 2, 3, 4
ROLE_ACT, ROLE_WEIGHT, ROLE_GRAD = 0, 1, 2
OP_FWD, OP_DGRAD, OP_WGRAD = 0, 1, 2


class MqConvError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} ({_status_string(status)})")


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
            "mqconv_codes_bytes": (S, [I, I, I32, I32, I32, I32]),
            "mqconv_scales_bytes": (S, [I, I32, I32, I32, I32, I32]),
            "mqconv_im2col_codes_bytes": (S, [CV, I]),
            "mqconv_im2col_scales_bytes": (S, [CV, I32]),
            "mqconv_quantize": (I, [P, mq_mx, P]),
            "mqconv_quantize_group": (I, [I32, P, ctypes.POINTER(mq_mx), P]),
            "mqconv_cbf_im2col": (I, [CV, mq_mx, P, P, P]),
            "mqconv_workspace_bytes": (S, [CV, I, I, I]),
            "mqconv_forward": (I, [CV, mq_mx, mq_mx, P, P, S, P]),
            "mqconv_forward_mx": (I, [CV, mq_mx, mq_mx, mq_mx, P, S, P]),
            "mqconv_backward_data": (I, [CV, mq_mx, mq_mx, P, P, S, P]),
            "mqconv_backward_data_mx": (I, [CV, mq_mx, mq_mx, mq_mx, P, S, P]),
            "mqconv_backward_weight": (I, [CV, mq_mx, mq_mx, P, P, S, P]),
            "mqconv_naive_workspace_bytes": (S, [CV, I, I, I]),
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


EXPORTED = ("mqconv_abi_version", "mqconv_status_string", "mqconv_codes_bytes", "mqconv_scales_bytes",
            "mqconv_im2col_codes_bytes", "mqconv_im2col_scales_bytes", "mqconv_quantize", "mqconv_quantize_group",
            "mqconv_cbf_im2col", "mqconv_workspace_bytes", "mqconv_forward", "mqconv_forward_mx", "mqconv_backward_data",
            "mqconv_backward_data_mx", "mqconv_backward_weight", "mqconv_naive_workspace_bytes", "mqconv_naive_forward",
            "mqconv_naive_backward_data", "mqconv_naive_backward_weight")


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

    def c_struct(self) -> mq_mx:
        return mq_mx(_ptr(self.codes), _ptr(self.scales), self.fmt, self.bp, self.role, *self.dims)


def mqconv_abi_version() -> int:
    return lib().mqconv_abi_version()


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


def mqconv_quantize(src, dst: MxTensor, stream=None) -> None:
    _check(lib().mqconv_quantize(_ptr(src), dst.c_struct(), _stream(stream)), "mqconv_quantize")


QUANTIZE_GROUP_MAX = 8


def mqconv_quantize_group(pairs, stream=None) -> None:
    """mqconv_quantize of several (src, dst MxTensor) pairs in one call."""
    pairs = list(pairs)
    n = len(pairs)
    srcs = (ctypes.c_void_p * max(1, n))(*[_ptr(p[0]) for p in pairs])
    dsts = (mq_mx * max(1, n))(*[p[1].c_struct() for p in pairs])
    _check(lib().mqconv_quantize_group(n, srcs, dsts, _stream(stream)), "mqconv_quantize_group")


def mqconv_cbf_im2col(shape, xq: MxTensor, col_codes, col_scales, stream=None) -> None:
    _check(lib().mqconv_cbf_im2col(ctypes.byref(_conv(shape)), xq.c_struct(), _ptr(col_codes),
                                   _ptr(col_scales), _stream(stream)), "mqconv_cbf_im2col")


def mqconv_workspace_bytes(shape, op: int, fa: int, fb: int) -> int:
    return lib().mqconv_workspace_bytes(ctypes.byref(_conv(shape)), op, fa, fb)


def _ws(ws):
    if ws is None:
        return None, 0
    return _ptr(ws), ws.numel() * ws.element_size()


def mqconv_forward(shape, xq: MxTensor, wq: MxTensor, y, ws=None, stream=None) -> None:
    p, n = _ws(ws)
    _check(lib().mqconv_forward(ctypes.byref(_conv(shape)), xq.c_struct(), wq.c_struct(), _ptr(y), p, n,
                                _stream(stream)), "mqconv_forward")


def mqconv_forward_mx(shape, xq: MxTensor, wq: MxTensor, yq: MxTensor, ws=None, stream=None) -> None:
    p, n = _ws(ws)
    _check(lib().mqconv_forward_mx(ctypes.byref(_conv(shape)), xq.c_struct(), wq.c_struct(), yq.c_struct(), p, n,
                                   _stream(stream)), "mqconv_forward_mx")


def mqconv_backward_data(shape, dyq: MxTensor, wq: MxTensor, dx, ws=None, stream=None) -> None:
    p, n = _ws(ws)
    _check(lib().mqconv_backward_data(ctypes.byref(_conv(shape)), dyq.c_struct(), wq.c_struct(), _ptr(dx), p,
                                      n, _stream(stream)), "mqconv_backward_data")


def mqconv_backward_data_mx(shape, dyq: MxTensor, wq: MxTensor, dxq: MxTensor, ws=None, stream=None) -> None:
    p, n = _ws(ws)
    _check(lib().mqconv_backward_data_mx(ctypes.byref(_conv(shape)), dyq.c_struct(), wq.c_struct(), dxq.c_struct(),
                                         p, n, _stream(stream)), "mqconv_backward_data_mx")


def mqconv_backward_weight(shape, dyq: MxTensor, xq: MxTensor, dw, ws=None, stream=None) -> None:
    p, n = _ws(ws)
    _check(lib().mqconv_backward_weight(ctypes.byref(_conv(shape)), dyq.c_struct(), xq.c_struct(), _ptr(dw),
                                        p, n, _stream(stream)), "mqconv_backward_weight")


def mqconv_naive_workspace_bytes(shape, op: int, fa: int, fb: int) -> int:
    return lib().mqconv_naive_workspace_bytes(ctypes.byref(_conv(shape)), op, fa, fb)


def mqconv_naive_forward(shape, x, w, fx: int, fw: int, y, ws, stream=None) -> None:
    p, n = _ws(ws)
    _check(lib().mqconv_naive_forward(ctypes.byref(_conv(shape)), _ptr(x), _ptr(w), fx, fw, _ptr(y), p, n,
                                      _stream(stream)), "mqconv_naive_forward")


def mqconv_naive_backward_data(shape, dy, w, fdy: int, fw: int, dx, ws, stream=None) -> None:
    p, n = _ws(ws)
    _check(lib().mqconv_naive_backward_data(ctypes.byref(_conv(shape)), _ptr(dy), _ptr(w), fdy, fw, _ptr(dx),
                                            p, n, _stream(stream)), "mqconv_naive_backward_data")


def mqconv_naive_backward_weight(shape, dy, x, fdy: int, fx: int, dw, ws, stream=None) -> None:
    p, n = _ws(ws)
    _check(lib().mqconv_naive_backward_weight(ctypes.byref(_conv(shape)), _ptr(dy), _ptr(x), fdy, fx,
                                              _ptr(dw), p, n, _stream(stream)), "mqconv_naive_backward_weight")
