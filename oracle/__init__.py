"""CPU oracle for the MicroQonv training hot path.

TEST INFRASTRUCTURE: only the tests, the smoke check and the benchmark's CPU
baseline leg may import this package. It shares no code with the GPU library
and never calls it. The heavy loops live in plain C (mqref.c, fp64, OpenMP);
this wrapper marshals numpy arrays and composes the steps in the paper's
order. Source: "MicroQonv: Reshaping Convolution Tensors for Efficient
Microscaling in Training and Inference":
  quantize ........ §II-D, §III-A (E8M0 power-of-two block scale), §IV-B
                    (square blocks along both GEMM directions)
  quantize_sr ..... §III-A (stochastic rounding of the gradient), with the
                    Philox4x32-10 counter-based generator
  cbf_im2col ...... §IV-A, Fig. 3
  conv_* .......... §II-A Eqs. (1)-(3)
  naive_* ......... §II-C (classic im2col, kernel flattening, the three GEMMs
                    G_W = G_Y . X'^T, G_X' = W^T . G_Y) and §III-C (quantize
                    the im2col-expanded tensor along each GEMM direction)
  nvfp_* .......... §II-D / §III-A Eqs. (4)-(6): FP32 tensor scale, E4M3
                    block scales, 8 x 8 square blocks (§IV-B, B = 64)
  cuyckens_* ...... §III-C (the square-block method of [25] extended to
                    convolution: the im2col-expanded X' quantized once in
                    square blocks and saved for the backward pass)
  activation_mse .. §IV-D, Table II (per-element quantization error of the
                    activation under each method)
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mqref.c")
_LIB = os.path.join(_HERE, "libmqref.so")

ELEM_BITS = {0: 8, 1: 8, 2: 6, 3: 6, 4: 4}
ROLE_ACT, ROLE_WEIGHT, ROLE_GRAD = 0, 1, 2


def build(force: bool = False) -> str:
    """Compile mqref.c with gcc (C99, OpenMP) into libmqref.so."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-std=gnu99", "-O2", "-fopenmp", "-fPIC", "-shared",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        LL = ctypes.c_longlong
        I = ctypes.c_int
        D = ctypes.c_double
        sig = {
            "mqref_threads": (I, []),
            "mqref_elem_bits": (I, [I]),
            "mqref_elem_emax": (I, [I]),
            "mqref_elem_max": (D, [I]),
            "mqref_decode": (D, [I, I]),
            "mqref_encode": (I, [I, D]),
            "mqref_encode_array": (None, [I, P, LL, P]),
            "mqref_quantize_view": (LL, [I, I, P, LL, LL, LL, LL, P, P]),
            "mqref_philox4x32_10": (None, [P, P, P]),
            "mqref_sr_word": (ctypes.c_uint32, [ctypes.c_uint64, LL, LL]),
            "mqref_encode_sr": (I, [I, D, ctypes.c_uint32]),
            "mqref_quantize_view_sr": (LL, [I, I, P, LL, LL, LL, LL, ctypes.c_uint64, P, P]),
            "mqref_dequant_view": (None, [I, I, P, P, LL, LL, LL, LL, P]),
            "mqref_nvfp_quantize_view": (ctypes.c_float, [I, P, LL, LL, LL, LL, P, P]),
            "mqref_nvfp_dequant_view": (None, [I, P, P, ctypes.c_float, LL, LL, LL, LL, P]),
            "mqref_row_bytes": (LL, [I, LL]),
            "mqref_pack_rows": (None, [I, P, LL, LL, P]),
            "mqref_unpack_rows": (None, [I, P, LL, LL, P]),
            "mqref_cbf_im2col_codes": (None, [P, I, P, P, P, P]),
            "mqref_cbf_im2col_f32": (None, [P, P, P]),
            "mqref_classic_im2col": (None, [P, P, P]),
            "mqref_col2im": (None, [P, P, P]),
            "mqref_conv_fwd": (None, [P, P, P, P]),
            "mqref_conv_dgrad": (None, [P, P, P, P]),
            "mqref_conv_wgrad": (None, [P, P, P, P]),
            "mqref_conv_fwd_points": (None, [P, P, P, LL, P, P]),
            "mqref_conv_dgrad_points": (None, [P, P, P, LL, P, P]),
            "mqref_conv_wgrad_points": (None, [P, P, P, LL, P, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _cv(shape) -> np.ndarray:
    """mq_conv as 11 ints: n, cin, h, w, cout, kh, kw, sh, sw, ph, pw."""
    t = shape.as_tuple() if hasattr(shape, "as_tuple") else tuple(shape)
    return np.ascontiguousarray(np.array(t, dtype=np.int32))


def out_hw(shape):
    cv = _cv(shape)
    return (int(cv[2] + 2 * cv[9] - cv[5]) // int(cv[7]) + 1,
            int(cv[3] + 2 * cv[10] - cv[6]) // int(cv[8]) + 1)


# --------------------------------------------------------------------------
# Element codec
# --------------------------------------------------------------------------
def threads() -> int:
    """OpenMP threads the oracle's loops run on."""
    return lib().mqref_threads()


def decode(fmt: int, code: int) -> float:
    return lib().mqref_decode(fmt, int(code))


def encode(fmt: int, v: float) -> int:
    return lib().mqref_encode(fmt, float(v))


def encode_array(fmt: int, v) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float64).reshape(-1)
    out = np.empty(v.size, np.uint8)
    lib().mqref_encode_array(fmt, _p(v), v.size, _p(out))
    return out


def elem_emax(fmt: int) -> int:
    return lib().mqref_elem_emax(fmt)


def elem_max(fmt: int) -> float:
    return lib().mqref_elem_max(fmt)


# --------------------------------------------------------------------------
# Block quantization over the 4-D view [A][P][B][C] (see mqref.c)
# --------------------------------------------------------------------------
def quantize_view(fmt: int, bp: int, src: np.ndarray, A: int, P: int, B: int, C: int):
    """Returns (logical codes uint8 [A*P*B*C], scales uint8 [A][B][ceil(P/bp)][ceil(C/32)],
    number of element quantizations)."""
    src = np.ascontiguousarray(src, dtype=np.float32).reshape(-1)
    assert src.size == A * P * B * C
    codes = np.empty(src.size, np.uint8)
    scales = np.empty(A * B * (-(-P // bp)) * (-(-C // 32)), np.uint8)
    n = lib().mqref_quantize_view(fmt, bp, _p(src), A, P, B, C, _p(codes), _p(scales))
    return codes, scales.reshape(A, B, -(-P // bp), -(-C // 32)), int(n)


def philox4x32_10(ctr, key):
    """Philox4x32-10 (Salmon et al., SC'11) of a 4-word counter and 2-word key."""
    c = np.ascontiguousarray(np.asarray(ctr, np.uint32))
    k = np.ascontiguousarray(np.asarray(key, np.uint32))
    out = np.empty(4, np.uint32)
    lib().mqref_philox4x32_10(_p(c), _p(k), _p(out))
    return out


def sr_word(seed: int, row: int, c: int) -> int:
    return int(lib().mqref_sr_word(seed, row, c))


def encode_sr(fmt: int, v: float, r: int) -> int:
    """Code of an already-scaled value rounded stochastically with random word r."""
    return lib().mqref_encode_sr(fmt, float(v), int(r))


def quantize_view_sr(fmt: int, bp: int, src: np.ndarray, A: int, P: int, B: int, C: int, seed: int):
    """quantize_view with stochastic rounding of the elements (§III-A)."""
    src = np.ascontiguousarray(src, dtype=np.float32).reshape(-1)
    assert src.size == A * P * B * C
    codes = np.empty(src.size, np.uint8)
    scales = np.empty(A * B * (-(-P // bp)) * (-(-C // 32)), np.uint8)
    n = lib().mqref_quantize_view_sr(fmt, bp, _p(src), A, P, B, C, seed, _p(codes), _p(scales))
    return codes, scales.reshape(A, B, -(-P // bp), -(-C // 32)), int(n)


def dequant_view(fmt: int, bp: int, codes: np.ndarray, scales: np.ndarray, A, P, B, C):
    codes = np.ascontiguousarray(codes, dtype=np.uint8).reshape(-1)
    scales = np.ascontiguousarray(scales, dtype=np.uint8).reshape(-1)
    out = np.empty(A * P * B * C, np.float64)
    lib().mqref_dequant_view(fmt, bp, _p(codes), _p(scales), A, P, B, C, _p(out))
    return out


def _role_view(role: int, dims):
    d0, d1, d2, d3 = dims
    if role in (ROLE_ACT, ROLE_GRAD):  # [H][W][N][C]: partner N
        return d0 * d1, d2, 1, d3
    return 1, d0, d1 * d2, d3  # WEIGHT [Cout][Kh][Kw][Cin]: partner Cout


def quantize(role: int, fmt: int, bp: int, x: np.ndarray):
    """Quantize a role-layout tensor once. Returns (logical codes shaped like
    x, scales shaped per the role's scale layout, count)."""
    dims = x.shape
    A, P, B, C = _role_view(role, dims)
    codes, scales, n = quantize_view(fmt, bp, x, A, P, B, C)
    if role in (ROLE_ACT, ROLE_GRAD):
        scales = scales.reshape(dims[0], dims[1], -(-dims[2] // bp), -(-dims[3] // 32))
    else:
        scales = scales.reshape(dims[1], dims[2], -(-dims[0] // bp), -(-dims[3] // 32))
    return codes.reshape(dims), scales, n


def quantize_sr(role: int, fmt: int, bp: int, x: np.ndarray, seed: int):
    """quantize() with stochastic rounding of the elements (the gradient's
    rounding in §III-A); the random word of an element is that of its memory
    row and channel (mqref.c, mqref_sr_word)."""
    dims = x.shape
    A, P, B, C = _role_view(role, dims)
    codes, scales, n = quantize_view_sr(fmt, bp, x, A, P, B, C, seed)
    if role in (ROLE_ACT, ROLE_GRAD):
        scales = scales.reshape(dims[0], dims[1], -(-dims[2] // bp), -(-dims[3] // 32))
    else:
        scales = scales.reshape(dims[1], dims[2], -(-dims[0] // bp), -(-dims[3] // 32))
    return codes.reshape(dims), scales, n


def dequantize(role: int, fmt: int, bp: int, codes: np.ndarray, scales: np.ndarray):
    dims = codes.shape
    A, P, B, C = _role_view(role, dims)
    return dequant_view(fmt, bp, codes, scales, A, P, B, C).reshape(dims)


# --------------------------------------------------------------------------
# Packed byte layout (runs of 32 codes)
# --------------------------------------------------------------------------
def row_bytes(fmt: int, C: int) -> int:
    return int(lib().mqref_row_bytes(fmt, C))


def pack(fmt: int, logical: np.ndarray) -> np.ndarray:
    """Pack logical codes [..., C] into [..., row_bytes]."""
    C = logical.shape[-1]
    rows = logical.size // C
    lg = np.ascontiguousarray(logical, dtype=np.uint8)
    out = np.empty(rows * row_bytes(fmt, C), np.uint8)
    lib().mqref_pack_rows(fmt, _p(lg), rows, C, _p(out))
    return out.reshape(logical.shape[:-1] + (row_bytes(fmt, C),))


def unpack(fmt: int, packed: np.ndarray, C: int) -> np.ndarray:
    rb = row_bytes(fmt, C)
    pk = np.ascontiguousarray(packed, dtype=np.uint8).reshape(-1)
    rows = pk.size // rb
    out = np.empty(rows * C, np.uint8)
    lib().mqref_unpack_rows(fmt, _p(pk), rows, C, _p(out))
    return out.reshape(packed.shape[:-1] + (C,)) if packed.ndim > 1 else out


def quantize_packed(role: int, fmt: int, bp: int, x: np.ndarray):
    """Quantize and pack: (packed codes [..., row_bytes], scales)."""
    codes, scales, _ = quantize(role, fmt, bp, x)
    return pack(fmt, codes), scales


# --------------------------------------------------------------------------
# Channel-batch-first im2col (§IV-A)
# --------------------------------------------------------------------------
def cbf_im2col_codes(shape, bp: int, xcodes: np.ndarray, xscales: np.ndarray):
    """Logical codes [H][W][N][C] + scales [H][W][nb][ncb] ->
    codes [Ho][Wo][N][Kh][Kw][C], scales [Ho][Wo][Kh][Kw][nb][ncb]."""
    cv = _cv(shape)
    N, C, KH, KW = int(cv[0]), int(cv[1]), int(cv[5]), int(cv[6])
    Ho, Wo = out_hw(shape)
    nb, ncb = -(-N // bp), -(-C // 32)
    oc = np.empty((Ho, Wo, N, KH, KW, C), np.uint8)
    os_ = np.empty((Ho, Wo, KH, KW, nb, ncb), np.uint8)
    xc = np.ascontiguousarray(xcodes, dtype=np.uint8)
    xs = np.ascontiguousarray(xscales, dtype=np.uint8)
    lib().mqref_cbf_im2col_codes(_p(cv), bp, _p(xc), _p(xs), _p(oc), _p(os_))
    return oc, os_


def cbf_im2col_f32(shape, x: np.ndarray) -> np.ndarray:
    cv = _cv(shape)
    N, C, KH, KW = int(cv[0]), int(cv[1]), int(cv[5]), int(cv[6])
    Ho, Wo = out_hw(shape)
    out = np.empty((Ho, Wo, N, KH, KW, C), np.float32)
    lib().mqref_cbf_im2col_f32(_p(cv), _p(np.ascontiguousarray(x, np.float32)), _p(out))
    return out


def quantize_im2col_expanded(shape, fmt: int, bp: int, xcol: np.ndarray):
    """Quantize an expanded CBF tensor [Ho][Wo][N][Kh][Kw][C] with the same
    block rule (32 channels x bp samples inside one (ho, wo, kh, kw))."""
    Ho, Wo, N, KH, KW, C = xcol.shape
    codes, scales, n = quantize_view(fmt, bp, xcol, Ho * Wo, N, KH * KW, C)
    return codes.reshape(xcol.shape), scales.reshape(Ho, Wo, KH, KW, -(-N // bp), -(-C // 32)), n


# --------------------------------------------------------------------------
# Direct convolution (Eqs. 1-3) on CBF fp64 tensors
# --------------------------------------------------------------------------
def _nchw(t):  # [H][W][N][C] -> [N][C][H][W]
    return np.ascontiguousarray(np.transpose(t, (2, 3, 0, 1)), dtype=np.float64)


def _cbf(t):  # [N][C][H][W] -> [H][W][N][C]
    return np.ascontiguousarray(np.transpose(t, (2, 3, 0, 1)))


def _w_oihw(w):  # [Cout][Kh][Kw][Cin] -> [Cout][Cin][Kh][Kw]
    return np.ascontiguousarray(np.transpose(w, (0, 3, 1, 2)), dtype=np.float64)


def _w_ohwi(w):
    return np.ascontiguousarray(np.transpose(w, (0, 2, 3, 1)))


def conv_fwd(shape, x, w):
    """x [H][W][N][Cin], w [Cout][Kh][Kw][Cin] -> y [Ho][Wo][N][Cout] (fp64)."""
    cv = _cv(shape)
    Ho, Wo = out_hw(shape)
    y = np.empty((int(cv[0]), int(cv[4]), Ho, Wo), np.float64)
    lib().mqref_conv_fwd(_p(cv), _p(_nchw(x)), _p(_w_oihw(w)), _p(y))
    return _cbf(y)


def conv_dgrad(shape, dy, w):
    cv = _cv(shape)
    dx = np.empty((int(cv[0]), int(cv[1]), int(cv[2]), int(cv[3])), np.float64)
    lib().mqref_conv_dgrad(_p(cv), _p(_nchw(dy)), _p(_w_oihw(w)), _p(dx))
    return _cbf(dx)


def conv_wgrad(shape, dy, x):
    cv = _cv(shape)
    dw = np.empty((int(cv[4]), int(cv[1]), int(cv[5]), int(cv[6])), np.float64)
    lib().mqref_conv_wgrad(_p(cv), _p(_nchw(dy)), _p(_nchw(x)), _p(dw))
    return _w_ohwi(dw)


class PointEvaluator:
    """Single outputs of the three operations on large problems. Holds the
    dequantized operands in NCHW fp64 once. Index tuples use the CBF naming:
      fwd (ho, wo, n, co); dgrad (h, w, n, ci); wgrad (co, kh, kw, ci)."""

    def __init__(self, shape, x=None, w=None, dy=None):
        self.cv = _cv(shape)
        self.x = _nchw(x) if x is not None else None
        self.w = _w_oihw(w) if w is not None else None
        self.dy = _nchw(dy) if dy is not None else None

    def fwd(self, pts):
        idx = np.ascontiguousarray(np.asarray(pts, np.int32)[:, [2, 3, 0, 1]])
        out = np.empty(len(idx), np.float64)
        lib().mqref_conv_fwd_points(_p(self.cv), _p(self.x), _p(self.w), len(idx), _p(idx), _p(out))
        return out

    def dgrad(self, pts):
        idx = np.ascontiguousarray(np.asarray(pts, np.int32)[:, [2, 3, 0, 1]])
        out = np.empty(len(idx), np.float64)
        lib().mqref_conv_dgrad_points(_p(self.cv), _p(self.dy), _p(self.w), len(idx), _p(idx), _p(out))
        return out

    def wgrad(self, pts):
        idx = np.ascontiguousarray(np.asarray(pts, np.int32)[:, [0, 3, 1, 2]])
        out = np.empty(len(idx), np.float64)
        lib().mqref_conv_wgrad_points(_p(self.cv), _p(self.dy), _p(self.x), len(idx), _p(idx), _p(out))
        return out


# --------------------------------------------------------------------------
# MicroQonv path: quantize once, CBF im2col on codes, three GEMMs (§IV)
# --------------------------------------------------------------------------
def microqonv_step(shape, x, w, dy, fx, fw, fdy, bp, passes=("fwd", "dgrad", "wgrad")):
    """Reference results of one training step on the dequantized operands."""
    out = {}
    xc, xs, _ = quantize(ROLE_ACT, fx, bp, x)
    wc, ws, _ = quantize(ROLE_WEIGHT, fw, bp, w)
    xh = dequantize(ROLE_ACT, fx, bp, xc, xs)
    wh = dequantize(ROLE_WEIGHT, fw, bp, wc, ws)
    out.update(xcodes=xc, xscales=xs, wcodes=wc, wscales=ws)
    if "fwd" in passes:
        out["y"] = conv_fwd(shape, xh, wh)
    if dy is not None and ("dgrad" in passes or "wgrad" in passes):
        gc, gs, _ = quantize(ROLE_GRAD, fdy, bp, dy)
        gh = dequantize(ROLE_GRAD, fdy, bp, gc, gs)
        out.update(dycodes=gc, dyscales=gs)
        if "dgrad" in passes:
            out["dx"] = conv_dgrad(shape, gh, wh)
        if "wgrad" in passes:
            out["dw"] = conv_wgrad(shape, gh, xh)
    return out


# --------------------------------------------------------------------------
# Naive path (§II-C, §III-C): im2col first, 1-D blocks of 32 along each GEMM
# direction, every tensor quantized twice
# --------------------------------------------------------------------------
def classic_im2col(shape, x):
    """X'[m][k], m = (ho, wo, n), k = (ci, kh, kw) channel-major."""
    cv = _cv(shape)
    Ho, Wo = out_hw(shape)
    M, K = Ho * Wo * int(cv[0]), int(cv[1]) * int(cv[5]) * int(cv[6])
    out = np.empty((M, K), np.float32)
    lib().mqref_classic_im2col(_p(cv), _p(np.ascontiguousarray(x, np.float32)), _p(out))
    return out


def col2im(shape, gcol):
    cv = _cv(shape)
    gx = np.empty((int(cv[2]), int(cv[3]), int(cv[0]), int(cv[1])), np.float64)
    lib().mqref_col2im(_p(cv), _p(np.ascontiguousarray(gcol, np.float64)), _p(gx))
    return gx


def flatten_kernel(w):
    """W_f[co][k], k = (ci, kh, kw) channel-major (§II-C2)."""
    return np.ascontiguousarray(np.transpose(w, (0, 3, 1, 2)).reshape(w.shape[0], -1))


def quantize_lines(fmt: int, mat: np.ndarray):
    """Quantize a matrix [R][L] in line blocks of 32 along each row; return
    the dequantized matrix (fp64) and the number of element quantizations."""
    R, L = mat.shape
    codes, scales, n = quantize_view(fmt, 1, mat, R, 1, 1, L)
    return dequant_view(fmt, 1, codes, scales, R, 1, 1, L).reshape(R, L), n


def naive_fwd(shape, x, w, fx, fw):
    """Y[m][co] = sum_k Q_k(X')[m][k] Q_k(W_f)[co][k]; returns ([Ho][Wo][N][Cout], count)."""
    Ho, Wo = out_hw(shape)
    xq, n1 = quantize_lines(fx, classic_im2col(shape, x))
    wq, n2 = quantize_lines(fw, flatten_kernel(w))
    y = xq @ wq.T
    return y.reshape(Ho, Wo, shape.n, shape.cout), {"A": n1, "W": n2}


def naive_dgrad(shape, dy, w, fdy, fw):
    """G_X' = Q_co(G_Y) . Q_co(W_f) then col2im; returns ([H][W][N][Cin], counts)."""
    M = dy.shape[0] * dy.shape[1] * dy.shape[2]
    gq, n1 = quantize_lines(fdy, dy.reshape(M, -1))
    wtq, n2 = quantize_lines(fw, np.ascontiguousarray(flatten_kernel(w).T))  # [k][co]
    gcol = gq @ wtq.T  # [m][k]
    return col2im(shape, gcol), {"G": n1, "W": n2}


def naive_wgrad(shape, dy, x, fdy, fx):
    """G_W = Q_m(G_Y)^T . Q_m(X'); returns ([Cout][Kh][Kw][Cin], counts)."""
    M = dy.shape[0] * dy.shape[1] * dy.shape[2]
    gtq, n1 = quantize_lines(fdy, np.ascontiguousarray(dy.reshape(M, -1).T))  # [co][m]
    xtq, n2 = quantize_lines(fx, np.ascontiguousarray(classic_im2col(shape, x).T))  # [k][m]
    dwf = gtq @ xtq.T  # [co][k], k = (ci, kh, kw)
    dw = dwf.reshape(shape.cout, shape.cin, shape.kh, shape.kw)
    return np.ascontiguousarray(np.transpose(dw, (0, 2, 3, 1))), {"G": n1, "A": n2}


# --------------------------------------------------------------------------
# Square-block comparator (§III-C): the method of [25], written for fully
# connected layers, extended to convolution by quantizing the im2col-expanded
# X' once in square blocks (32 rows x 32 columns here, the block the MFMA
# scale granularity allows), W_f and G_Y once in square blocks too; the same
# codes serve the GEMM along either direction, so nothing is quantized twice,
# but X' is stored expanded.
# --------------------------------------------------------------------------
def quantize_squares(fmt: int, mat: np.ndarray):
    """Quantize a matrix [R][L] in 32 x 32 square blocks (32 consecutive rows x
    32 consecutive columns, truncated at the edges). Returns (logical codes
    [R][L], scales [ceil(R/32)][ceil(L/32)], count)."""
    R, L = mat.shape
    codes, scales, n = quantize_view(fmt, 32, mat, 1, R, 1, L)
    return codes.reshape(R, L), scales.reshape(-(-R // 32), -(-L // 32)), n


def dequant_squares(fmt: int, codes: np.ndarray, scales: np.ndarray):
    R, L = codes.shape
    return dequant_view(fmt, 32, codes, scales, 1, R, 1, L).reshape(R, L)


def cuyckens_im2col_quantize(shape, x, fx):
    """X' = classic im2col of x [M][K] (k = (ci, kh, kw)), quantized once in
    square blocks: (codes [M][K], scales [M/32][K/32], count = |X'|)."""
    return quantize_squares(fx, classic_im2col(shape, x))


def cuyckens_fwd(shape, xcodes, xscales, w, fx, fw):
    """Y[m][co] = sum_k X'q[m][k] W_fq[co][k] on the saved X'q; W_f in squares."""
    Ho, Wo = out_hw(shape)
    xq = dequant_squares(fx, xcodes, xscales)
    wc, ws_, n = quantize_squares(fw, flatten_kernel(w))
    y = xq @ dequant_squares(fw, wc, ws_).T
    return y.reshape(Ho, Wo, shape.n, shape.cout), {"W": n}


def cuyckens_dgrad(shape, dy, w, fdy, fw):
    """G_X' = G_Yq . W_fq (both square-quantized once), then col2im."""
    M = dy.shape[0] * dy.shape[1] * dy.shape[2]
    gc, gs, n1 = quantize_squares(fdy, dy.reshape(M, -1))
    wc, ws_, n2 = quantize_squares(fw, flatten_kernel(w))
    gcol = dequant_squares(fdy, gc, gs) @ dequant_squares(fw, wc, ws_)  # [m][k]
    return col2im(shape, gcol), {"G": n1, "W": n2}


def cuyckens_wgrad(shape, dy, xcodes, xscales, fdy, fx):
    """G_W = G_Yq^T . X'q on the saved X'q; returns [Cout][Kh][Kw][Cin]."""
    M = dy.shape[0] * dy.shape[1] * dy.shape[2]
    gc, gs, n = quantize_squares(fdy, dy.reshape(M, -1))
    dwf = dequant_squares(fdy, gc, gs).T @ dequant_squares(fx, xcodes, xscales)  # [co][k]
    dwr = dwf.reshape(shape.cout, shape.cin, shape.kh, shape.kw)
    return np.ascontiguousarray(np.transpose(dwr, (0, 2, 3, 1))), {"G": n}


def activation_mse(shape, x, fmt, method, bp=32):
    """Mean squared error per element between every activation value a GEMM
    consumes and its fp32 value (Table II's per-element quantization MSE),
    over the values the forward and the weight-gradient GEMMs read:
      "microqonv": X quantized once (32 channels x bp samples per pixel); each
                   value of X' is a copy of one of them;
      "naive":     X' quantized in lines of 32 along k (forward) and along m
                   (weight gradient), both uses counted;
      "cuyckens":  X' quantized once in 32 x 32 squares.
    Padding positions of X' (zeros, exact in every method) are left out."""
    xf = np.asarray(x, np.float32)
    xcol = classic_im2col(shape, xf).astype(np.float64)
    ids = classic_im2col(shape, (np.arange(xf.size, dtype=np.float64).reshape(xf.shape) + 1).astype(np.float32))
    inside = ids > 0
    if method == "microqonv":
        c, s, _ = quantize(ROLE_ACT, fmt, bp, xf)
        xq = dequantize(ROLE_ACT, fmt, bp, c, s).astype(np.float32)
        err = (classic_im2col(shape, xq).astype(np.float64) - xcol)[inside]
        return float(np.mean(err ** 2))
    if method == "cuyckens":
        c, s, _ = quantize_squares(fmt, xcol.astype(np.float32))
        err = (dequant_squares(fmt, c, s) - xcol)[inside]
        return float(np.mean(err ** 2))
    fq, _ = quantize_lines(fmt, xcol.astype(np.float32))
    bq, _ = quantize_lines(fmt, np.ascontiguousarray(xcol.T).astype(np.float32))
    e1 = (fq - xcol)[inside]
    e2 = (bq.T - xcol)[inside]
    return float((np.sum(e1 ** 2) + np.sum(e2 ** 2)) / (e1.size + e2.size))


# --------------------------------------------------------------------------
# Two-level (NVFP-style) scaling, Eqs. (4)-(6) (see mqref.c)
# --------------------------------------------------------------------------
def nvfp_quantize(role: int, fmt: int, x: np.ndarray):
    """Returns (logical codes shaped like x, E4M3 block scales
    [A][B][ceil(P/8)][ceil(C/8)] of the role's view, fp32 tensor scale T)."""
    dims = x.shape
    A, P, B, C = _role_view(role, dims)
    src = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
    codes = np.empty(src.size, np.uint8)
    bs = np.empty(A * B * (-(-P // 8)) * (-(-C // 8)), np.uint8)
    T = lib().mqref_nvfp_quantize_view(fmt, _p(src), A, P, B, C, _p(codes), _p(bs))
    return codes.reshape(dims), bs.reshape(A, B, -(-P // 8), -(-C // 8)), float(np.float32(T))


def nvfp_dequantize(role: int, fmt: int, codes: np.ndarray, bscales: np.ndarray, T: float):
    dims = codes.shape
    A, P, B, C = _role_view(role, dims)
    out = np.empty(codes.size, np.float64)
    lib().mqref_nvfp_dequant_view(fmt, _p(np.ascontiguousarray(codes, np.uint8).reshape(-1)),
                                  _p(np.ascontiguousarray(bscales, np.uint8).reshape(-1)), T, A, P, B, C, _p(out))
    return out.reshape(dims)
